// layout.h — host-side canvas layout produced by the example packer.
//
// Plain C++ (no HIP): the packer is integer host code. The device copy of a
// layout (rectangles, per-example offsets, unit schedule, eid/border maps) is
// described by DescOffsets; abi.cpp uploads it.
#pragma once

#include <cstdint>
#include <string>
#include <vector>

#if defined(__HIPCC__)
#define MDL_HD __host__ __device__
#else
#define MDL_HD
#endif

namespace mdl {

// Geometry of one example's local anti-diagonals. For an example of h x w
// cells and a scan direction, a cell with direction-local coordinates (a, b)
// (a = rows already scanned above it, b = columns already scanned before it)
// lies on diagonal s = a + b; diagonal s holds the cells a in [lo(s), lo(s)+len(s)).
// The per-direction stash stores an example's cells diagonal after diagonal,
// each diagonal in increasing a, so cell (a, b) sits at start(s) + a - lo(s).
MDL_HD inline int dg_len(int h, int w, int s) {
    int m = h < w ? h : w;
    int v = s + 1;
    if (v > m) v = m;
    int t = h + w - 1 - s;
    return v < t ? v : t;
}
MDL_HD inline int dg_lo(int /*h*/, int w, int s) { return s - w + 1 > 0 ? s - w + 1 : 0; }
MDL_HD inline int64_t dg_start(int h, int w, int s) {
    int A = h < w ? h : w, B = h < w ? w : h;
    if (s <= A) return (int64_t)s * (s + 1) / 2;
    if (s <= B) return (int64_t)A * (A + 1) / 2 + (int64_t)(s - A) * A;
    int64_t t = (int64_t)h + w - 1 - s;
    return (int64_t)h * w - t * (t + 1) / 2;
}

// Weight-gradient work split (see Layout::segs): at most kGroups groups (each one task per direction), at
// least about kGroupMinCells cells each, at most kGroupSegs segments each; from kGroupRound groups on, a
// multiple of kGroupRound (whole rounds of tasks on a 256-CU device at two workgroups per unit).
constexpr int kGroups = 512;
constexpr int kGroupMinCells = 512;
constexpr int kGroupRound = 128;
constexpr int kGroupSegs = 16;
// Direction-sum chunks (see Layout::dsum): runs of at most kSumChunk real pixels of one example.
constexpr int kSumChunk = 256;

struct DescOffsets {
    size_t rect = 0;      // int32 [n][4] computed region (y0, x0, h, w)
    size_t real = 0;      // int32 [n][4] real pixels
    size_t flat_off = 0;  // int64 [n+1] prefix of real pixels (flat per-example tensors)
    size_t cell_off = 0;  // int64 [n+1] prefix of computed cells (per-direction stash)
    size_t units = 0;     // int32 [4n] (example*4 + direction), most cells first
    size_t segs = 0;      // int32 [nsegs][3] (example, first cell, end cell) of the weight-gradient split
    size_t groups = 0;    // int32 [ngroups+1] first segment of each weight-gradient workgroup
    size_t gorder = 0;    // int32 [4 ngroups] the weight-gradient tasks (4 group + direction) in readiness order
    size_t dsum = 0;      // int32 [nsum][3] direction-sum chunks (example, first pixel, end pixel) in readiness order
    size_t eid = 0;       // int32 [Hc*Wc]
    size_t border = 0;    // uint8 [Hc*Wc]
    size_t total = 0;
};

struct Layout {
    int32_t n = 0, Hc = 0, Wc = 0, mode = 0, sep = 0, canvas_w_min = 0;
    std::vector<int32_t> rect;   // [n][4]
    std::vector<int32_t> real;   // [n][4]
    std::vector<std::vector<int32_t>> rows;
    std::vector<int64_t> flat_off, cell_off;
    std::vector<int32_t> units;
    std::vector<int32_t> eid;    // host maps
    std::vector<uint8_t> border;
    int64_t real_pixels = 0, computed_cells = 0;
    int32_t max_depth = 0, max_diag = 0;
    // Weight-gradient split: the computed cells of all examples (example order, row-major within
    // one) cut into ranges of nearly equal size, one per workgroup; a range's pieces inside one
    // example are its segments (cells [first, end) of the region). groups[g] .. groups[g+1] are
    // workgroup g's segments. The partial sums are per workgroup and per segment (for kernels that
    // take one segment per workgroup), so nparts() = max(nsegs, ngroups) partial blocks.
    std::vector<int32_t> segs;
    std::vector<int32_t> groups;
    // the weight-gradient tasks (task 4 g + d: direction d of group g) ordered by the largest dependent-step
    // count (h + w - 1) of the group's examples, ties by task index: the order in which they become ready
    // while the reverse wavefront runs (its units all start together)
    std::vector<int32_t> gorder;
    // the direction sum's chunks: runs of at most kSumChunk real pixels (row-major in the example's real
    // region), the examples in the order their forward units finish (fewest dependent steps first, ties
    // by index), each example's chunks in pixel order
    std::vector<int32_t> dsum;
    int32_t nsegs = 0, ngroups = 0, nsum = 0;
    int64_t nparts() const { return nsegs > ngroups ? nsegs : ngroups; }
    DescOffsets off;
    std::vector<uint8_t> host_desc;  // descriptor bytes up to off.eid (the maps are built on device)
};

// Returns 0 or a negative MDL_E* code with `err` set.
int build_layout(const int32_t* heights, const int32_t* widths, int32_t n, int32_t canvas_w_min,
                 int32_t sep, int32_t mode, Layout& out, std::string& err);

}  // namespace mdl

struct mdl_layout {
    mdl::Layout L;
};
