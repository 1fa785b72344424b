// kernels.h — device view of a layout and the launchers of the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <tuple>
#include <utility>

#include "layout.h"

namespace mdl {

// Launch timing. While a clock is installed on the calling thread, every
// launch below hands the dispatch a pair of events that record its own start
// and end (hipExtLaunchKernel), so timing inserts no marker packets between
// kernels and the elapsed time is the kernel's alone.
struct LaunchClock {
    virtual ~LaunchClock() = default;
    virtual void events(hipEvent_t* start, hipEvent_t* stop) = 0;
};
extern thread_local LaunchClock* t_launch_clock;

// Launches `kernel` with its arguments converted to the kernel's own
// parameter types; the launch status is left for hipGetLastError.
template <typename... P, typename... A>
inline void launch(void (*kernel)(P...), dim3 grid, dim3 block, size_t lds, hipStream_t st, A&&... args) {
    static_assert(sizeof...(P) == sizeof...(A), "kernel argument count");
    std::tuple<P...> vals(static_cast<P>(std::forward<A>(args))...);
    std::apply(
        [&](auto&... v) {
            void* argv[] = {static_cast<void*>(&v)...};
            hipEvent_t a = nullptr, b = nullptr;
            if (t_launch_clock) t_launch_clock->events(&a, &b);
            if (a && b)
                (void)hipExtLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, argv, lds, st, a, b, 0);
            else
                (void)hipLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, argv, lds, st);
        },
        vals);
}

// Pointers into an uploaded descriptor plus the sizes the kernels need.
struct Dev {
    const int32_t* rect;      // [n][4] computed region (y0, x0, h, w)
    const int32_t* real;      // [n][4] real pixels
    const int64_t* flat_off;  // [n+1]
    const int64_t* cell_off;  // [n+1]
    const int32_t* units;     // [4n]
    const int32_t* segs;      // [nsegs][3] (example, first cell, end cell)
    const int32_t* groups;    // [ngroups+1] first segment of each weight-gradient workgroup
    const int32_t* gorder;    // [4 ngroups] the weight-gradient tasks (4 group + direction) in readiness order
    const int32_t* dsum;      // [nsum][3] direction-sum chunks (example, first pixel, end pixel) in readiness order
    int32_t* eid;             // [Hc*Wc]
    uint8_t* border;          // [Hc*Wc]
    int n, Hc, Wc;
    int64_t T;                // computed cells per direction
    int64_t N;                // real pixels
    int max_depth, max_diag;
    int nsegs, ngroups, nsum;
};

// Canvas position of the direction-local cell (a, b) of an example whose
// computed region is (y0, x0, h, w), for direction d (bit 1: rows scanned
// bottom-up, bit 0: columns scanned right-to-left).
struct Flip {
    int y0, x0, h, w;
    bool fy, fx;
    MDL_HD int y(int a) const { return y0 + (fy ? h - 1 - a : a); }
    MDL_HD int x(int b) const { return x0 + (fx ? w - 1 - b : b); }
};

// Decode a cell's position in an example's diagonal-major order: index q ->
// (diagonal s, row a). Inverse of dg_start(s) + a - dg_lo(s).
MDL_HD inline void dg_decode(int h, int w, int64_t q, int& s, int& a) {
    const int A = h < w ? h : w, B = h < w ? w : h;
    const int64_t t1 = (int64_t)A * (A + 1) / 2;
    const int64_t t2 = t1 + (int64_t)(B - A) * A;
    if (q < t1) {
        int v = (int)((sqrt(8.0 * (double)q + 1.0) - 1.0) * 0.5);
        while ((int64_t)v * (v + 1) / 2 > q) --v;
        while ((int64_t)(v + 1) * (v + 2) / 2 <= q) ++v;
        s = v;
    } else if (q < t2) {
        s = A + (int)((q - t1) / A);
    } else {
        const int64_t r = (int64_t)h * w - 1 - q;  // position counted from the last cell
        int v = (int)((sqrt(8.0 * (double)r + 1.0) - 1.0) * 0.5);
        while ((int64_t)v * (v + 1) / 2 > r) --v;
        while ((int64_t)(v + 1) * (v + 2) / 2 <= r) ++v;
        s = h + w - 2 - v;
    }
    a = dg_lo(h, w, s) + (int)(q - dg_start(h, w, s));
}

// Largest e with off[e] <= g (off has n+1 ascending entries, off[0] = 0).
MDL_HD inline int find_example(const int64_t* off, int n, int64_t g) {
    int lo = 0, hi = n - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (off[mid] <= g) lo = mid; else hi = mid - 1;
    }
    return lo;
}

// Workspace carving for one MDLSTM layer (all offsets 256-byte aligned).
// Projection and stash layouts. For direction d, computed cell t (each
// example's cells in diagonal-major order, examples one after another) and
// hidden unit k, with T computed cells per direction:
//   Z4[((d*T + t)*H + k)*4 + g]  pre-activation x.Wx + b of gate g = i, f_l, f_u, o
//   Z1[(d*T + t)*H + k]          pre-activation of the cell input g
//   SA[((d*T + t)*H + k)*4 + m]  gate values i, f_l, f_u, o
//   SB[((d*T + t)*H + k)*4 + m]  the cell input g, tanh(c), and the predecessors' memory states c_l, c_u
//                                (everything the reverse wavefront's factors need: bwd_factors in devmath.h)
//   dA4, dA1: the gate pre-activation gradients in the layout of Z4 / Z1
// A lane owning (cell, k) reads or writes each four-value group with one
// 16-byte access. Z1 follows Z4 in the workspace's projection region, SB
// follows SA in its stash region (at z1_offset). The skewed-schedule kernels
// keep their own stash in the same region: gates i, f_l, f_u, o at SA's place
// and (g, c) pairs, [(d*T + t)*H + k][2], at SB's.
MDL_HD inline int64_t z1_offset(int64_t T, int H) { return 4 * T * 4 * (int64_t)H; }

struct WsLayout {
    size_t stash = 0;   // float [4][T][8H]: SA then SB, the forward values of every cell the reverse wavefront needs
    size_t zda = 0;     // float [4][T][5H]: projection x.Wx+b (forward), gate gradients dA (backward)
    size_t part = 0;    // float [nparts][4][(C+1+2H)*5H]: weight-gradient partial sums
    size_t dxp = 0;     // float [4][T][C]: each direction's share of the input gradient
    size_t flags = 0;   // int32 [4n + 8 ngroups + kFlagTail]: the weight-gradient overlap's flags (OverlapFlags)
    size_t fflags = 0;  // int32 [4n + 2 nsum + kFlagTail]: the direction sum's overlap with the forward (OverlapFlags)
    size_t total = 0;
    int64_t nparts = 0;
};
constexpr int kFlagTail = 16;
WsLayout ws_layout(int64_t T, int64_t nparts, int C, int H, int64_t nflags, int64_t nfflags);
// the flags and counters of the weight gradient's overlap with the reverse wavefront, in the workspace's
// flags region ([4n] done, [4 ngroups] taken, [4 ngroups] abandoned, then the four single counters), all zero
// before the reverse wavefront
struct OverlapFlags {
    int32_t* done;       // [4n] set when reverse-wavefront unit (example, direction) has stored its gate gradients
    int32_t* taken;      // [4 ngroups] set by the workgroup that takes queue position i (beside or after)
    int32_t* abandoned;  // [4 ngroups] tasks claimed beside the wavefront but not ready in time, to do afterwards
    int32_t* queue;      // the next position of gorder to claim
    int32_t* stop;       // set once a group was not ready in time: the launch beside the wavefront claims no more
    int32_t* nab;        // entries of `abandoned`
    int32_t* abq;        // the next entry of `abandoned` to claim
};
// how a launch of the claiming weight-gradient kernel takes its groups
enum WgClaim : int {
    kClaimBeside = 0,     // beside the reverse wavefront: wait (bounded) for each task's units to finish
    kClaimDrain = 1,      // after the reverse wavefront on its stream: one workgroup per queue position not taken
    kClaimAbandoned = 2,  // after both: the tasks given up beside the wavefront
};

// launchers: return hipSuccess or the launch error
hipError_t launch_build_maps(const Dev& D, hipStream_t st);
// n ints set to v by a kernel (no memset node, so a captured graph replays it as a kernel)
hipError_t launch_fill_i32(int32_t* p, int64_t n, int32_t v, hipStream_t st);
hipError_t launch_zero_outside(const Dev& D, float* buf, int K, int planes, hipStream_t st);
hipError_t launch_scatter(const Dev& D, const void* x_flat, int C, int dtype, void* x_canvas, hipStream_t st);
hipError_t launch_projection(const Dev& D, const void* x_canvas, int dtype, int C, int H, const float* Wx,
                             const float* b, float* Z, hipStream_t st);
size_t fwd_chain_lds(int H, int Lmax);
size_t bwd_chain_lds(int H, int Lmax);
int chain_max_items();
bool chain_uses_mfma(int H, int Lmax);
// forward wavefront with the input projection fused, recurrent product on the f16 matrix cores
// (split operands, fp32-class accuracy); supported for the instantiated (H, C, dtype) combinations
bool fwd16_supported(int H, int C, int dtype, int Lmax);
size_t fwd16_lds(int H, int C, int dtype, int Lmax);
// done (may be null): [4n] flags, unit (example e, direction d) sets done[4e + d] once its h stores are visible
hipError_t launch_fwd16(const Dev& D, const void* x_canvas, int dtype, int C, int H, const float* Wx,
                        const float* b, const float* Ul, const float* Uu, float* stash, float* h_dirs,
                        int32_t* done, hipStream_t st);
// reverse wavefront on the f16 matrix cores (split, power-of-two scaled operands)
bool bwd16_supported(int H, int Lmax);
size_t bwd16_lds(int H, int Lmax);
// done (may be null): [4n] flags, unit (example e, direction d) sets done[4e + d] once its stores are visible
hipError_t launch_bwd16(const Dev& D, int H, const float* Ul, const float* Uu, const float* stash,
                        const float* dy_flat, const float* dh_dirs, float* dA, int32_t* done, hipStream_t st);
// wavefront kernels for small hidden sizes (H <= 10) on the vector ALUs, fp32, input projection fused
bool small_fwd_supported(int H, int C, int dtype, int Lmax);
bool small_bwd_supported(int H, int Lmax);
size_t small_fwd_lds(int H, int Lmax);
size_t small_bwd_lds(int H, int Lmax);
hipError_t launch_fwd_small(const Dev& D, const void* x_canvas, int dtype, int C, int H, const float* Wx,
                            const float* b, const float* Ul, const float* Uu, float* stash, float* h_dirs,
                            hipStream_t st);
hipError_t launch_bwd_small(const Dev& D, int H, const float* Ul, const float* Uu, const float* stash,
                            const float* dy_flat, const float* dh_dirs, float* dA, hipStream_t st);
hipError_t launch_fwd_chain(const Dev& D, int H, const float* Ul, const float* Uu, const float* Z,
                            float* stash, float* h_dirs, hipStream_t st);
hipError_t launch_dirsum(const Dev& D, const float* h_dirs, int H, float* y_flat, hipStream_t st);
// the direction sum in the layout's chunks (D.dsum), for the overlap with the forward: whether the chunked
// form runs for these buffers (4-wide vectors), and its launches, taking chunks from the claim queue in F as
// launch_wgrad2_claim takes tasks (kClaimBeside: waits, bounded by `budget`, until the example's four forward
// units are flagged in F.done; kClaimDrain: one workgroup per queue position not taken; kClaimAbandoned).
// lds_hold: LDS bytes each workgroup of the beside launch holds (at least its own): enough that it cannot share
// a compute unit with a wavefront workgroup
bool dirsum_chunked_supported(const Dev& D, const float* h_dirs, int H, const float* y_flat);
hipError_t launch_dirsum_claim(const Dev& D, const float* h_dirs, int H, float* y_flat, const OverlapFlags& F,
                               WgClaim mode, int workgroups, long long budget, size_t lds_hold, hipStream_t st);
hipError_t launch_bwd_chain(const Dev& D, int H, const float* Ul, const float* Uu, const float* stash,
                            const float* dy_flat, const float* dh_dirs, float* dA, hipStream_t st);
// software-pipelined weight-gradient kernel for the instantiated (C, H, dtype) shapes
bool wgrad2_supported(int C, int H, int dtype);
size_t wgrad2_lds_bytes(int C, int H, int dtype);
// tasks (group, direction) into part[group][d] and, when dxp is not null, each direction's share of dx into
// dxp [4][T][C] (cells numbered as in the layout's cell offsets, row-major inside each region)
hipError_t launch_wgrad2(const Dev& D, const void* x_canvas, int dtype, int C, int H, const float* h_dirs,
                         const float* dA, const float* Wx, float* part, float* dxp, hipStream_t st);
// the same tasks taken from the claim queue in F (in the layout's readiness order): beside the wavefront and
// from the abandoned list by `workgroups` workgroups that loop until there is none left (beside, each wait for
// a task's units, flagged in F.done, is bounded by `budget` shader-clock cycles); after the wavefront by one
// workgroup per queue position whose taken flag is still clear (`workgroups` and `budget` unused); lds_hold as
// for launch_dirsum_claim
hipError_t launch_wgrad2_claim(const Dev& D, const void* x_canvas, int dtype, int C, int H, const float* h_dirs,
                               const float* dA, const float* Wx, float* part, float* dxp, const OverlapFlags& F,
                               WgClaim mode, int workgroups, long long budget, size_t lds_hold, hipStream_t st);
// dx from the four directions' shares in dxp (added in direction order): dx_flat at the real pixels,
// dx_canvas at the computed cells (zero outside the real pixels); nothing when both are null
hipError_t launch_dx_sum(const Dev& D, int C, const float* dxp, float* dx_flat, float* dx_canvas, hipStream_t st);
size_t wgrad_lds_bytes(int C, int H);
// dxp: the workspace's dx-share region (used by the shapes launch_wgrad2 supports)
hipError_t launch_wgrad(const Dev& D, const void* x_canvas, int dtype, int C, int H, const float* h_dirs,
                        const float* dA, const float* Wx, float* part, float* dxp, float* dWx, float* dUl, float* dUu,
                        float* db, float* dx_flat, float* dx_canvas, hipStream_t st);
// the sum of nparts partial blocks [nparts][4][C+1+2H][5H] into dWx, dUl, dUu, db
hipError_t launch_wgrad_reduce(int64_t nparts, int C, int H, const float* part, float* dWx, float* dUl, float* dUu,
                               float* db, hipStream_t st);
hipError_t launch_conv_fwd(const Dev& Dk, const Dev& Dk1, const float* h_dirs_k, int H, int kh, int kw,
                           const float* Wc, const float* bc, int Cout, float* x_k1, hipStream_t st);
int64_t conv_nchunks(const Dev& Dk1);
// the Leaky LP cell (k_leaky.hip): forward and reverse wavefronts on the fp32 matrix cores, and the weight
// gradients of its memory-state projections (partials in `part`, added in workgroup order)
bool leaky_supported(int H, int C, int Lmax);
size_t leaky_fwd_lds(int H, int Lmax);
size_t leaky_bwd_lds(int H, int Lmax);
hipError_t launch_fwd_leaky(const Dev& D, const void* x_canvas, int dtype, int C, int H, const float* Wx,
                            const float* b, const float* Ul, const float* Uu, const float* Vl, const float* Vu,
                            float* stash, float* h_dirs, hipStream_t st);
hipError_t launch_bwd_leaky(const Dev& D, int H, const float* Ul, const float* Uu, const float* Vl, const float* Vu,
                            const float* stash, const float* dy_flat, const float* dh_dirs, float* dA,
                            hipStream_t st);
hipError_t launch_dv_leaky(const Dev& D, int H, const float* stash, const float* dA, float* part, float* dVl,
                           float* dVu, hipStream_t st);
// the pages' schedule (k_skew.hip): one launch per column of the input-skewed canvas, Hc + Wc - 1 per pass
bool skew_supported(int H);
int skew_columns(const Dev& D);
hipError_t launch_skew_fwd(const Dev& D, int H, const float* Ul, const float* Uu, const float* Z, float* stash,
                           float* h_dirs, hipStream_t st);
hipError_t launch_skew_bwd(const Dev& D, int H, const float* Ul, const float* Uu, const float* stash,
                           const float* dy_flat, const float* dh_dirs, float* dA, float* dcb, hipStream_t st);
// this device's fixed weight-gradient scratch of the block conv (address and size), for callers that cannot
// allocate; every call on one device shares it
hipError_t conv_scratch(void** ptr, size_t* bytes);
size_t conv_fwd_lds(int H, int kh, int kw, int Cout);
size_t conv_wgrad_lds(int H, int kh, int kw, int Cout);
size_t conv_data_lds(int H, int kh, int kw, int Cout);
hipError_t launch_conv_bwd(const Dev& Dk, const Dev& Dk1, const float* h_dirs_k, int H, int kh, int kw,
                           const float* Wc, int Cout, const float* dx_k1, float* dh_k, float* dWc,
                           float* dbc, float* part, hipStream_t st);

// model head (height collapse, shared fully-connected layer, CTC loss); workspace sizes in floats
struct CtcWs {
    int64_t smax = 0;   // states of the longest blank-padded label, 2 Umax + 1
    int64_t slot = 0;   // per-example slot (a multiple of 4 floats): the arrays of ctc_offsets
    int64_t part = 0;   // offset of the per-example weight-gradient partials
    int64_t total = 0;
};
// offsets (floats, each a multiple of 4) of one example's arrays after w0 leading floats: Y [Tmax][H],
// log-probabilities and dz [Tmax][K] (float), log alpha and log beta [Tmax][smax] (double), then the
// blank-padded label (smax ints) where the arrays sit in LDS
struct CtcOff {
    int64_t y, ly, dz, la, lb, lp;
};
MDL_HD inline int64_t ctc_al4(int64_t v) { return (v + 3) & ~int64_t(3); }
MDL_HD inline CtcOff ctc_offsets(int64_t w0, int Tmax, int H, int K, int64_t smax) {
    CtcOff o;
    o.y = ctc_al4(w0);
    o.ly = ctc_al4(o.y + (int64_t)Tmax * H);
    o.dz = ctc_al4(o.ly + (int64_t)Tmax * K);
    o.la = ctc_al4(o.dz + (int64_t)Tmax * K);
    o.lb = o.la + 2 * (int64_t)Tmax * smax;
    o.lp = ctc_al4(o.lb + 2 * (int64_t)Tmax * smax);
    return o;
}
MDL_HD inline CtcWs ctc_ws(int n, int Tmax, int H, int K, int Umax) {
    CtcWs w;
    w.smax = 2 * (int64_t)Umax + 1;
    w.slot = ctc_offsets(0, Tmax, H, K, w.smax).lp;
    w.part = (int64_t)n * w.slot;
    w.total = w.part + (int64_t)n * ((int64_t)H + 1) * K;
    return w;
}
// LDS bytes of the head kernel's in-LDS form; the launcher takes it when it fits lds_limit
size_t ctc_lds_bytes(int Tmax, int H, int K, int Umax);
hipError_t launch_ctc_head(const Dev& D, const float* y_flat, int H, const float* Wfc, const float* bfc, int K,
                           const int32_t* labels, const int32_t* label_off, int64_t nlab, int Umax, int Tmax,
                           float* ws, float* loss, float* dy_flat, float* dW, float* db, size_t lds_limit,
                           hipStream_t st);

}  // namespace mdl
