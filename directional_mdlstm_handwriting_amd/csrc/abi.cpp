// abi.cpp — the extern "C" entry points of libmdlstm: argument checks, workspace
// carving and kernel launches. Every check runs before the first launch, so a
// failing call writes nothing; errors never cross the ABI as exceptions.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstring>
#include <new>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/mdlstm.h"
#include "kernels.h"
#include "leaky16.h"
#include "layout.h"

namespace mdl {
thread_local LaunchClock* t_launch_clock = nullptr;
}  // namespace mdl

namespace {

thread_local std::string g_err;

int fail(int code, const std::string& msg) {
    g_err = msg;
    return code;
}

int hip_fail(hipError_t e, const char* where) {
    return fail(MDL_EHIP, std::string(where) + ": " + hipGetErrorString(e));
}
int hip_fail(hipError_t e, const std::string& where) { return hip_fail(e, where.c_str()); }

const mdl::Layout& L_of(const mdl_layout* l) { return l->L; }

// ints of the workspace's flags region: the overlap's per-unit and per-task flags and its counters
int64_t nflags_of(const mdl::Layout& L) { return 4 * (int64_t)L.n + 8 * (int64_t)L.ngroups + mdl::kFlagTail; }
// ints of the workspace's forward flags region: the direction sum's overlap with the forward
int64_t nfflags_of(const mdl::Layout& L) { return 4 * (int64_t)L.n + 2 * (int64_t)L.nsum + mdl::kFlagTail; }

// the weight-gradient overlap: 1 on (default), 0 off, 2 on with no time to wait for any task (every task
// claimed beside the wavefront is given up and done after it); a stream (default priority) and fork / join
// events per device
std::atomic<int> g_overlap{1};
struct Side {
    hipStream_t s = nullptr;
    hipEvent_t fork = nullptr, join = nullptr;
    int ncu = 0;
};
constexpr int kMaxSideDevices = 64;
int side_of(Side*& out) {
    static std::mutex mu;
    static Side sides[kMaxSideDevices];
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "mdl_backward: current device");
    if (dev < 0 || dev >= kMaxSideDevices) return fail(MDL_EUNSUPPORTED, "mdl_backward: device index above 63");
    std::lock_guard<std::mutex> lk(mu);
    Side& sd = sides[dev];
    if (sd.s == nullptr) {
        Side n;
        if ((e = hipDeviceGetAttribute(&n.ncu, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess ||
            (e = hipStreamCreateWithFlags(&n.s, hipStreamNonBlocking)) != hipSuccess ||
            (e = hipEventCreateWithFlags(&n.fork, hipEventDisableTiming)) != hipSuccess ||
            (e = hipEventCreateWithFlags(&n.join, hipEventDisableTiming)) != hipSuccess)
            return hip_fail(e, "mdl_backward: weight-gradient stream");
        sd = n;
    }
    out = &sd;
    return MDL_OK;
}

mdl::Dev make_dev(const mdl_layout* lay, const void* d_desc) {
    const mdl::Layout& L = L_of(lay);
    const uint8_t* b = static_cast<const uint8_t*>(d_desc);
    mdl::Dev D;
    D.rect = reinterpret_cast<const int32_t*>(b + L.off.rect);
    D.real = reinterpret_cast<const int32_t*>(b + L.off.real);
    D.flat_off = reinterpret_cast<const int64_t*>(b + L.off.flat_off);
    D.cell_off = reinterpret_cast<const int64_t*>(b + L.off.cell_off);
    D.units = reinterpret_cast<const int32_t*>(b + L.off.units);
    D.segs = reinterpret_cast<const int32_t*>(b + L.off.segs);
    D.groups = reinterpret_cast<const int32_t*>(b + L.off.groups);
    D.gorder = reinterpret_cast<const int32_t*>(b + L.off.gorder);
    D.dsum = reinterpret_cast<const int32_t*>(b + L.off.dsum);
    D.eid = reinterpret_cast<int32_t*>(const_cast<uint8_t*>(b + L.off.eid));
    D.border = const_cast<uint8_t*>(b + L.off.border);
    D.n = L.n;
    D.Hc = L.Hc;
    D.Wc = L.Wc;
    D.T = L.computed_cells;
    D.N = L.real_pixels;
    D.max_depth = L.max_depth;
    D.max_diag = L.max_diag;
    D.nsegs = L.nsegs;
    D.ngroups = L.ngroups;
    D.nsum = L.nsum;
    return D;
}

// LDS each workgroup of a launch beside a wavefront holds so that it cannot share a compute unit with one of the
// wavefront's workgroups (whose LDS is wave_lds, out of lmax per compute unit): those would then take the compute
// unit's issue slots from the wavefront's dependent chain, or, placed first, keep a wavefront workgroup waiting
size_t beside_lds_hold(size_t lmax, size_t wave_lds) { return wave_lds < lmax ? lmax - wave_lds + 256 : 0; }

int max_lds(size_t& out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    int v = 0;
    e = hipDeviceGetAttribute(&v, hipDeviceAttributeMaxSharedMemoryPerBlock, dev);
    if (e != hipSuccess) return hip_fail(e, "hipDeviceGetAttribute");
    out = (size_t)v;
    return MDL_OK;
}

int check_layer(const char* fn, const mdl_layout* layout, const void* d_desc, int32_t C, int32_t H, int32_t x_dtype) {
    if (!layout || !d_desc) return fail(MDL_EINVAL, std::string(fn) + ": null layout or descriptor");
    if (C < 1 || H < 1) return fail(MDL_EINVAL, std::string(fn) + ": need C >= 1 and H >= 1");
    if (x_dtype != MDL_F32 && x_dtype != MDL_BF16) return fail(MDL_EINVAL, std::string(fn) + ": unknown dtype");
    if (C > 1024 || H > 1024) return fail(MDL_EUNSUPPORTED, std::string(fn) + ": C or H above 1024");
    const mdl::Layout& L = L_of(layout);
    const int64_t P = (int64_t)L.Hc * L.Wc;
    if (P * 4 * std::max(H, C) >= (int64_t(1) << 40)) return fail(MDL_EOVERFLOW, std::string(fn) + ": canvas too large");
    return MDL_OK;
}

// ---- optional per-launch event timing ---------------------------------------------------------
struct TimedLaunch {
    std::string name;
    std::vector<hipEvent_t> ev;  // start, stop of each dispatch of the group, in launch order
};
bool g_timing = false;
std::string g_timing_only;  // empty: every group
std::mutex g_tmu;
std::vector<TimedLaunch> g_tlog;
std::vector<hipEvent_t> g_event_pool;

hipEvent_t take_event() {
    if (!g_event_pool.empty()) {
        hipEvent_t e = g_event_pool.back();
        g_event_pool.pop_back();
        return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
}

// While timing is on, installs itself as the thread's launch clock for one launcher call: each dispatch
// gets a start/stop event pair recorded by the dispatch itself, and the group's time runs from the first
// dispatch's start to the last one's stop.
class Timed : public mdl::LaunchClock {
  public:
    explicit Timed(const char* name) : name_(name) {
        if (!g_timing || (!g_timing_only.empty() && g_timing_only != name)) return;
        prev_ = mdl::t_launch_clock;
        mdl::t_launch_clock = this;
        on_ = true;
    }
    ~Timed() override {
        if (!on_) return;
        mdl::t_launch_clock = prev_;
        if (ev_.empty()) return;
        std::lock_guard<std::mutex> lk(g_tmu);
        g_tlog.push_back({name_, std::move(ev_)});
    }
    void events(hipEvent_t* start, hipEvent_t* stop) override {
        std::lock_guard<std::mutex> lk(g_tmu);
        hipEvent_t a = take_event(), b = take_event();
        if (!a || !b) {
            if (a) g_event_pool.push_back(a);
            if (b) g_event_pool.push_back(b);
            return;
        }
        ev_.push_back(a);
        ev_.push_back(b);
        *start = a;
        *stop = b;
    }

  private:
    const char* name_;
    bool on_ = false;
    mdl::LaunchClock* prev_ = nullptr;
    std::vector<hipEvent_t> ev_;
};

#define GUARD_BEGIN try {
#define GUARD_END                                                      \
    }                                                                  \
    catch (const std::bad_alloc&) { return fail(MDL_ENOMEM, "out of host memory"); } \
    catch (...) { return fail(MDL_EINVAL, "unexpected internal error"); }

}  // namespace

extern "C" {

int mdl_pack(const int32_t* heights, const int32_t* widths, int32_t n, int32_t canvas_w_min, int32_t sep,
             int32_t mode, mdl_layout** out) {
    GUARD_BEGIN
    if (!out) return fail(MDL_EINVAL, "mdl_pack: null output pointer");
    *out = nullptr;
    mdl_layout* lay = new (std::nothrow) mdl_layout;
    if (!lay) return fail(MDL_ENOMEM, "mdl_pack: out of host memory");
    std::string err;
    const int rc = mdl::build_layout(heights, widths, n, canvas_w_min, sep, mode, lay->L, err);
    if (rc != MDL_OK) {
        delete lay;
        return fail(rc, err);
    }
    *out = lay;
    return MDL_OK;
    GUARD_END
}

int mdl_pack_level(const mdl_layout* lk, int32_t kh, int32_t kw, int32_t canvas_w_min, int32_t sep, int32_t mode,
                   mdl_layout** out) {
    GUARD_BEGIN
    if (!out) return fail(MDL_EINVAL, "mdl_pack_level: null output pointer");
    *out = nullptr;
    if (!lk) return fail(MDL_EINVAL, "mdl_pack_level: null layout");
    if (kh < 1 || kw < 1) return fail(MDL_EINVAL, "mdl_pack_level: block sizes must be positive");
    const mdl::Layout& A = L_of(lk);
    // the block-strided convolution covers each example with ceil(h / kh) x ceil(w / kw) blocks, the last
    // row and column of blocks padded with zeros
    std::vector<int32_t> hs(A.n), ws(A.n);
    for (int e = 0; e < A.n; ++e) {
        hs[e] = (A.real[4 * e + 2] + kh - 1) / kh;
        ws[e] = (A.real[4 * e + 3] + kw - 1) / kw;
    }
    return mdl_pack(hs.data(), ws.data(), A.n, canvas_w_min, sep, mode, out);
    GUARD_END
}

void mdl_layout_free(mdl_layout* layout) { delete layout; }

int mdl_layout_info(const mdl_layout* layout, int64_t* info) {
    if (!layout || !info) return fail(MDL_EINVAL, "mdl_layout_info: null argument");
    const mdl::Layout& L = L_of(layout);
    info[MDL_INFO_N] = L.n;
    info[MDL_INFO_CANVAS_H] = L.Hc;
    info[MDL_INFO_CANVAS_W] = L.Wc;
    info[MDL_INFO_ROWS] = (int64_t)L.rows.size();
    info[MDL_INFO_REAL_PIXELS] = L.real_pixels;
    info[MDL_INFO_COMPUTED_CELLS] = L.computed_cells;
    info[MDL_INFO_MAX_DEPTH] = L.max_depth;
    info[MDL_INFO_MAX_DIAG] = L.max_diag;
    info[MDL_INFO_MODE] = L.mode;
    info[MDL_INFO_WG_GROUPS] = L.ngroups;
    return MDL_OK;
}

int mdl_layout_rects(const mdl_layout* layout, int32_t* rects, int32_t* real) {
    if (!layout) return fail(MDL_EINVAL, "mdl_layout_rects: null layout");
    const mdl::Layout& L = L_of(layout);
    if (rects) std::memcpy(rects, L.rect.data(), sizeof(int32_t) * 4 * L.n);
    if (real) std::memcpy(real, L.real.data(), sizeof(int32_t) * 4 * L.n);
    return MDL_OK;
}

int mdl_layout_rows(const mdl_layout* layout, int32_t* row_start, int32_t* row_examples) {
    if (!layout || !row_start || !row_examples) return fail(MDL_EINVAL, "mdl_layout_rows: null argument");
    const mdl::Layout& L = L_of(layout);
    int32_t k = 0;
    for (size_t r = 0; r < L.rows.size(); ++r) {
        row_start[r] = k;
        for (int32_t e : L.rows[r]) row_examples[k++] = e;
    }
    row_start[L.rows.size()] = k;
    return MDL_OK;
}

int mdl_layout_units(const mdl_layout* layout, int32_t* units, size_t* desc_offset) {
    if (!layout || !units || !desc_offset) return fail(MDL_EINVAL, "mdl_layout_units: null argument");
    const mdl::Layout& L = L_of(layout);
    std::copy(L.units.begin(), L.units.end(), units);
    *desc_offset = L.off.units;
    return MDL_OK;
}

int mdl_layout_maps(const mdl_layout* layout, int32_t* eid, uint8_t* border) {
    if (!layout) return fail(MDL_EINVAL, "mdl_layout_maps: null layout");
    const mdl::Layout& L = L_of(layout);
    if (eid) std::memcpy(eid, L.eid.data(), sizeof(int32_t) * L.eid.size());
    if (border) std::memcpy(border, L.border.data(), L.border.size());
    return MDL_OK;
}

int mdl_layout_device_size(const mdl_layout* layout, size_t* bytes, size_t* eid_offset, size_t* border_offset) {
    if (!layout || !bytes) return fail(MDL_EINVAL, "mdl_layout_device_size: null argument");
    const mdl::Layout& L = L_of(layout);
    *bytes = L.off.total;
    if (eid_offset) *eid_offset = L.off.eid;
    if (border_offset) *border_offset = L.off.border;
    return MDL_OK;
}

int mdl_layout_upload(const mdl_layout* layout, void* d_desc, size_t bytes, void* stream) {
    GUARD_BEGIN
    if (!layout || !d_desc) return fail(MDL_EINVAL, "mdl_layout_upload: null argument");
    const mdl::Layout& L = L_of(layout);
    if (bytes < L.off.total) return fail(MDL_ESIZE, "mdl_layout_upload: descriptor buffer too small");
    if (reinterpret_cast<uintptr_t>(d_desc) % 8) return fail(MDL_EINVAL, "mdl_layout_upload: descriptor not 8-byte aligned");
    hipStream_t st = static_cast<hipStream_t>(stream);
    hipError_t e = hipMemcpyAsync(d_desc, L.host_desc.data(), L.host_desc.size(), hipMemcpyHostToDevice, st);
    if (e != hipSuccess) return hip_fail(e, "mdl_layout_upload: copy");
    {
        Timed t("build_maps");
        e = mdl::launch_build_maps(make_dev(layout, d_desc), st);
    }
    if (e != hipSuccess) return hip_fail(e, "mdl_layout_upload: map kernels");
    e = hipStreamSynchronize(st);
    if (e != hipSuccess) return hip_fail(e, "mdl_layout_upload: synchronize");
    return MDL_OK;
    GUARD_END
}

int mdl_workspace_size(const mdl_layout* layout, int32_t C, int32_t H, size_t* bytes) {
    if (!layout || !bytes) return fail(MDL_EINVAL, "mdl_workspace_size: null argument");
    if (C < 1 || H < 1) return fail(MDL_EINVAL, "mdl_workspace_size: need C >= 1 and H >= 1");
    *bytes = mdl::ws_layout(L_of(layout).computed_cells, L_of(layout).nparts(), C, H, nflags_of(L_of(layout)), nfflags_of(L_of(layout))).total;
    return MDL_OK;
}

int mdl_scatter(const mdl_layout* layout, const void* d_desc, const void* x_flat, int32_t C, int32_t dtype,
                void* x_canvas, void* stream) {
    GUARD_BEGIN
    int rc = check_layer("mdl_scatter", layout, d_desc, C, 1, dtype);
    if (rc) return rc;
    if (!x_flat || !x_canvas) return fail(MDL_EINVAL, "mdl_scatter: null tensor");
    hipError_t e;
    {
        Timed t("scatter");
        e = mdl::launch_scatter(make_dev(layout, d_desc), x_flat, C, dtype, x_canvas, static_cast<hipStream_t>(stream));
    }
    if (e != hipSuccess) return hip_fail(e, "mdl_scatter");
    return MDL_OK;
    GUARD_END
}

// The kernels address device tensors through buffer descriptors with 32-bit byte ranges and offsets.
// The wavefront kernels take one direction's h plane and the canvas input each as one range and send a
// masked lane 2^30 bytes past its start; the gate stash is addressed one example at a time. The
// software-pipelined weight-gradient kernel takes one direction's h plane and gate gradients per range.
static int check_extent(const char* fn, const mdl::Layout& L, int C, int H, int x_dtype, bool backward) {
    const int64_t plane = (int64_t)L.Hc * L.Wc * H * 4;
    const int64_t xbytes = (int64_t)L.Hc * L.Wc * C * (x_dtype == MDL_BF16 ? 2 : 4);
    const int64_t dabytes = L.computed_cells * 5 * (int64_t)H * 4;  // one direction
    const int64_t lim = (int64_t(1) << 31) - 16;
    if (plane > (int64_t(1) << 30) || xbytes > (int64_t(1) << 30))
        return fail(MDL_EUNSUPPORTED, std::string(fn) + ": one direction's h plane or the canvas input above 1 GiB");
    if (backward && dabytes >= lim)
        return fail(MDL_EUNSUPPORTED, std::string(fn) + ": one direction's gate gradients above 2 GiB");
    // The wavefront kernels address one example's stash and gate gradients (at most 16 H bytes per cell) through
    // a per-example buffer range and park the accesses of idle lanes at byte offset 2^30, which must lie past
    // that range.
    int64_t cells = 0;
    for (int e = 0; e < L.n; ++e) cells = std::max<int64_t>(cells, (int64_t)L.rect[4 * e + 2] * L.rect[4 * e + 3]);
    if (cells * 16 * H > (int64_t(1) << 30))
        return fail(MDL_EUNSUPPORTED, std::string(fn) + ": one example's cells x 16 H bytes above 1 GiB");
    return MDL_OK;
}

static int check_cell(const char* fn, int32_t cell, const void* Vl, const void* Vu) {
    if (cell == MDL_CELL_MDLSTM) {
        if (Vl || Vu) return fail(MDL_EINVAL, std::string(fn) + ": memory-state projections given with the MDLSTM cell");
        return MDL_OK;
    }
    if (cell == MDL_CELL_LEAKY_LP) {
        if (!Vl || !Vu) return fail(MDL_EINVAL, std::string(fn) + ": the Leaky LP cell needs its memory-state projections");
        return MDL_OK;
    }
    return fail(MDL_EINVAL, std::string(fn) + ": unknown cell");
}

// The forward wavefront of mdl_forward and, when y_flat is given, the direction sum of mdl_dirsum_unpack.
// The sum overlaps the wavefront when its units leave at least half of the compute units free (f16 path,
// chunked sum supported): each unit flags itself when its h plane is stored, persistent workgroups on the
// library's second stream take the sum's chunks (in the order their examples finish) once all four of an
// example's units are done, and the launch after the wavefront takes the rest; every chunk runs the same code.
static int forward_impl(const char* fn, const mdl_layout* layout, const void* d_desc, const void* x_canvas,
                        int32_t x_dtype, int32_t C, int32_t H, int32_t cell, const float* Wx, const float* Ul,
                        const float* Uu, const float* b, const float* Vl, const float* Vu, float* h_dirs,
                        float* y_flat, void* ws, size_t ws_bytes, void* stream) {
    const std::string F(fn);
    int rc = check_layer(fn, layout, d_desc, C, H, x_dtype);
    if (rc) return rc;
    if ((rc = check_cell(fn, cell, Vl, Vu))) return rc;
    if (!x_canvas || !Wx || !Ul || !Uu || !b || !h_dirs || !ws) return fail(MDL_EINVAL, F + ": null tensor");
    const mdl::Layout& L = L_of(layout);
    const mdl::WsLayout W = mdl::ws_layout(L.computed_cells, L.nparts(), C, H, nflags_of(L), nfflags_of(L));
    if (ws_bytes < W.total) return fail(MDL_ESIZE, F + ": workspace smaller than mdl_workspace_size");
    if ((rc = check_extent(fn, L, C, H, x_dtype, false))) return rc;
    const mdl::Dev D = make_dev(layout, d_desc);
    hipStream_t st = static_cast<hipStream_t>(stream);
    uint8_t* wsb = static_cast<uint8_t*>(ws);
    float* stash = reinterpret_cast<float*>(wsb + W.stash);
    hipError_t e = hipSuccess;
    // the direction sum after the wavefront (when asked for and not overlapped)
    auto dirsum_after = [&]() -> int {
        if (!y_flat) return MDL_OK;
        Timed t("dirsum");
        const hipError_t e2 = mdl::launch_dirsum(D, h_dirs, H, y_flat, st);
        return e2 == hipSuccess ? MDL_OK : hip_fail(e2, F + ": direction sum");
    };
    if (cell == MDL_CELL_LEAKY_LP) {
        if (!mdl::leaky_supported(H, C, L.max_diag))
            return fail(MDL_EUNSUPPORTED, F + ": the Leaky LP cell runs for H in {4, 8, 16, 32}, C <= 16 and "
                                              "a widest diagonal of at most 64 cells (32 at H = 32)");
        size_t lmax = 0;
        if ((rc = max_lds(lmax))) return rc;
        if (mdl::leaky_fwd_lds(H, L.max_diag) > lmax) return fail(MDL_EUNSUPPORTED, F + ": diagonal state exceeds LDS");
        {
            Timed t("zero_fill");
            e = mdl::launch_zero_outside(D, h_dirs, H, 4, st);
        }
        if (e != hipSuccess) return hip_fail(e, F + ": zero fill");
        {
            Timed t("fwd_wavefront");
            e = mdl::launch_fwd_leaky(D, x_canvas, x_dtype, C, H, Wx, b, Ul, Uu, Vl, Vu, stash, h_dirs, st);
        }
        if (e != hipSuccess) return hip_fail(e, F + ": wavefront");
        return dirsum_after();
    }
    // small hidden sizes: vector-ALU wavefront; instantiated matrix-core shapes: f16 wavefront; both with
    // the projection fused. Otherwise the projection as its own GEMM and the general fp32 wavefront.
    const bool small = mdl::small_fwd_supported(H, C, x_dtype, L.max_diag);
    const bool fused = !small && mdl::fwd16_supported(H, C, x_dtype, L.max_diag);
    if (!small && !fused && (int64_t)L.max_diag * H > mdl::chain_max_items())
        return fail(MDL_EUNSUPPORTED, F + ": widest diagonal x H exceeds the wavefront kernel's items");
    size_t lmax = 0;
    if ((rc = max_lds(lmax))) return rc;
    const size_t need = small ? mdl::small_fwd_lds(H, L.max_diag)
                              : (fused ? mdl::fwd16_lds(H, C, x_dtype, L.max_diag) : mdl::fwd_chain_lds(H, L.max_diag));
    if (need > lmax) return fail(MDL_EUNSUPPORTED, F + ": recurrent weights and diagonal state exceed LDS");
    float* Z = reinterpret_cast<float*>(wsb + W.zda);
    if (!fused) {  // the f16 forward clears h outside the computed regions itself, in its smallest units' tail
        Timed t("zero_fill");
        e = mdl::launch_zero_outside(D, h_dirs, H, 4, st);
    }
    if (e != hipSuccess) return hip_fail(e, F + ": zero fill");
    Side* side = nullptr;
    int ov_wg = 0;
    const int ov_mode = g_overlap.load();
    if (fused && y_flat && ov_mode != 0 && mdl::dirsum_chunked_supported(D, h_dirs, H, y_flat)) {
        if ((rc = side_of(side))) return rc;
        const int free_cu = side->ncu - 4 * L.n;
        if (2 * free_cu >= side->ncu) ov_wg = std::min(free_cu, (int)L.nsum);
    }
    mdl::OverlapFlags Fl{};
    if (ov_wg > 0) {
        int32_t* fl = reinterpret_cast<int32_t*>(wsb + W.fflags);
        Fl.done = fl;
        Fl.taken = fl + 4 * L.n;
        Fl.abandoned = Fl.taken + L.nsum;
        Fl.queue = Fl.abandoned + L.nsum;
        Fl.stop = Fl.queue + 1;
        Fl.nab = Fl.queue + 2;
        Fl.abq = Fl.queue + 3;
        if ((e = mdl::launch_fill_i32(fl, nfflags_of(L), 0, st)) != hipSuccess)
            return hip_fail(e, F + ": overlap flags");
        if ((e = hipEventRecord(side->fork, st)) != hipSuccess || (e = hipStreamWaitEvent(side->s, side->fork, 0)) != hipSuccess)
            return hip_fail(e, F + ": fork to the library's stream");
    }
    if (small) {
        Timed t("fwd_wavefront");
        e = mdl::launch_fwd_small(D, x_canvas, x_dtype, C, H, Wx, b, Ul, Uu, stash, h_dirs, st);
    } else if (fused) {
        Timed t("fwd_wavefront");
        e = mdl::launch_fwd16(D, x_canvas, x_dtype, C, H, Wx, b, Ul, Uu, stash, h_dirs, ov_wg > 0 ? Fl.done : nullptr,
                              st);
    } else {
        {
            Timed t("projection");
            e = mdl::launch_projection(D, x_canvas, x_dtype, C, H, Wx, b, Z, st);
        }
        if (e != hipSuccess) return hip_fail(e, F + ": projection");
        Timed t("fwd_wavefront");
        e = mdl::launch_fwd_chain(D, H, Ul, Uu, Z, stash, h_dirs, st);
    }
    if (e != hipSuccess) return hip_fail(e, F + ": wavefront");
    if (ov_wg == 0) return dirsum_after();
    // each wait at most ~2^15 clock cycles per dependent step of the layout, at least 2^26 cycles
    const long long budget = ov_mode == 2 ? 0 : std::max<long long>(1ll << 26, (long long)L.max_depth << 15);
    {
        Timed t("dirsum_overlap");
        e = mdl::launch_dirsum_claim(D, h_dirs, H, y_flat, Fl, mdl::kClaimBeside, ov_wg, budget,
                                     beside_lds_hold(lmax, need), side->s);
    }
    if (e != hipSuccess) return hip_fail(e, F + ": direction sum beside the wavefront");
    if ((e = hipEventRecord(side->join, side->s)) != hipSuccess) return hip_fail(e, F + ": library's stream");
    {
        Timed t("dirsum");
        e = mdl::launch_dirsum_claim(D, h_dirs, H, y_flat, Fl, mdl::kClaimDrain, 0, 0, 0, st);
        if (e == hipSuccess && (e = hipStreamWaitEvent(st, side->join, 0)) == hipSuccess)
            e = mdl::launch_dirsum_claim(D, h_dirs, H, y_flat, Fl, mdl::kClaimAbandoned, 16, 0, 0, st);
    }
    if (e != hipSuccess) return hip_fail(e, F + ": direction sum");
    return MDL_OK;
}

int mdl_forward(const mdl_layout* layout, const void* d_desc, const void* x_canvas, int32_t x_dtype, int32_t C,
                int32_t H, int32_t cell, const float* Wx, const float* Ul, const float* Uu, const float* b,
                const float* Vl, const float* Vu, float* h_dirs, void* ws, size_t ws_bytes, void* stream) {
    GUARD_BEGIN
    return forward_impl("mdl_forward", layout, d_desc, x_canvas, x_dtype, C, H, cell, Wx, Ul, Uu, b, Vl, Vu, h_dirs,
                        nullptr, ws, ws_bytes, stream);
    GUARD_END
}

int mdl_forward_dirsum(const mdl_layout* layout, const void* d_desc, const void* x_canvas, int32_t x_dtype,
                       int32_t C, int32_t H, int32_t cell, const float* Wx, const float* Ul, const float* Uu,
                       const float* b, const float* Vl, const float* Vu, float* h_dirs, float* y_flat, void* ws,
                       size_t ws_bytes, void* stream) {
    GUARD_BEGIN
    if (!y_flat) return fail(MDL_EINVAL, "mdl_forward_dirsum: null tensor");
    return forward_impl("mdl_forward_dirsum", layout, d_desc, x_canvas, x_dtype, C, H, cell, Wx, Ul, Uu, b, Vl, Vu,
                        h_dirs, y_flat, ws, ws_bytes, stream);
    GUARD_END
}

static size_t skew_dcb_offset(const mdl::WsLayout& W) { return (W.total + 255) & ~size_t(255); }

int mdl_skewed_workspace_size(const mdl_layout* layout, int32_t C, int32_t H, size_t* bytes) {
    if (!layout || !bytes) return fail(MDL_EINVAL, "mdl_skewed_workspace_size: null argument");
    if (C < 1 || H < 1) return fail(MDL_EINVAL, "mdl_skewed_workspace_size: need C >= 1 and H >= 1");
    const mdl::Layout& L = L_of(layout);
    const mdl::WsLayout W = mdl::ws_layout(L.computed_cells, L.nparts(), C, H, nflags_of(L), nfflags_of(L));
    *bytes = skew_dcb_offset(W) + sizeof(float) * 4 * (size_t)L.computed_cells * 2 * H;
    return MDL_OK;
}

int mdl_forward_skewed(const mdl_layout* layout, const void* d_desc, const void* x_canvas, int32_t x_dtype,
                       int32_t C, int32_t H, const float* Wx, const float* Ul, const float* Uu, const float* b,
                       float* h_dirs, void* ws, size_t ws_bytes, void* stream) {
    GUARD_BEGIN
    int rc = check_layer("mdl_forward_skewed", layout, d_desc, C, H, x_dtype);
    if (rc) return rc;
    if (!x_canvas || !Wx || !Ul || !Uu || !b || !h_dirs || !ws)
        return fail(MDL_EINVAL, "mdl_forward_skewed: null tensor");
    if (!mdl::skew_supported(H)) return fail(MDL_EUNSUPPORTED, "mdl_forward_skewed: runs for H in {4, 16}");
    const mdl::Layout& L = L_of(layout);
    size_t need = 0;
    mdl_skewed_workspace_size(layout, C, H, &need);
    if (ws_bytes < need) return fail(MDL_ESIZE, "mdl_forward_skewed: workspace smaller than mdl_skewed_workspace_size");
    if ((rc = check_extent("mdl_forward_skewed", L, C, H, x_dtype, true))) return rc;
    const mdl::WsLayout W = mdl::ws_layout(L.computed_cells, L.nparts(), C, H, nflags_of(L), nfflags_of(L));
    const mdl::Dev D = make_dev(layout, d_desc);
    hipStream_t st = static_cast<hipStream_t>(stream);
    uint8_t* wsb = static_cast<uint8_t*>(ws);
    float* Z = reinterpret_cast<float*>(wsb + W.zda);
    float* stash = reinterpret_cast<float*>(wsb + W.stash);
    hipError_t e;
    {
        Timed t("zero_fill");
        e = mdl::launch_zero_outside(D, h_dirs, H, 4, st);
    }
    if (e != hipSuccess) return hip_fail(e, "mdl_forward_skewed: zero fill");
    {
        Timed t("projection");
        e = mdl::launch_projection(D, x_canvas, x_dtype, C, H, Wx, b, Z, st);
    }
    if (e != hipSuccess) return hip_fail(e, "mdl_forward_skewed: projection");
    {
        Timed t("fwd_skewed_columns");
        e = mdl::launch_skew_fwd(D, H, Ul, Uu, Z, stash, h_dirs, st);
    }
    if (e != hipSuccess) return hip_fail(e, "mdl_forward_skewed: column steps");
    return MDL_OK;
    GUARD_END
}

int mdl_backward_skewed(const mdl_layout* layout, const void* d_desc, const void* x_canvas, int32_t x_dtype,
                        int32_t C, int32_t H, const float* Wx, const float* Ul, const float* Uu, const float* h_dirs,
                        const float* dy_flat, const float* dh_dirs, float* dx_flat, float* dx_canvas, float* dWx,
                        float* dUl, float* dUu, float* db, void* ws, size_t ws_bytes, void* stream) {
    GUARD_BEGIN
    int rc = check_layer("mdl_backward_skewed", layout, d_desc, C, H, x_dtype);
    if (rc) return rc;
    if (!x_canvas || !Wx || !Ul || !Uu || !h_dirs || !ws || !dWx || !dUl || !dUu || !db)
        return fail(MDL_EINVAL, "mdl_backward_skewed: null tensor");
    if ((dy_flat == nullptr) == (dh_dirs == nullptr))
        return fail(MDL_EINVAL, "mdl_backward_skewed: pass exactly one of dy_flat and dh_dirs");
    if (!mdl::skew_supported(H)) return fail(MDL_EUNSUPPORTED, "mdl_backward_skewed: runs for H in {4, 16}");
    const mdl::Layout& L = L_of(layout);
    size_t need = 0;
    mdl_skewed_workspace_size(layout, C, H, &need);
    if (ws_bytes < need)
        return fail(MDL_ESIZE, "mdl_backward_skewed: workspace smaller than mdl_skewed_workspace_size");
    if ((rc = check_extent("mdl_backward_skewed", L, C, H, x_dtype, true))) return rc;
    const bool wg2 = mdl::wgrad2_supported(C, H, x_dtype);
    size_t lmax = 0;
    if ((rc = max_lds(lmax))) return rc;
    if ((wg2 ? mdl::wgrad2_lds_bytes(C, H, x_dtype) : mdl::wgrad_lds_bytes(C, H)) > lmax)
        return fail(MDL_EUNSUPPORTED, "mdl_backward_skewed: weight-gradient tile exceeds LDS");
    const mdl::WsLayout W = mdl::ws_layout(L.computed_cells, L.nparts(), C, H, nflags_of(L), nfflags_of(L));
    const mdl::Dev D = make_dev(layout, d_desc);
    hipStream_t st = static_cast<hipStream_t>(stream);
    uint8_t* wsb = static_cast<uint8_t*>(ws);
    float* dA = reinterpret_cast<float*>(wsb + W.zda);
    const float* stash = reinterpret_cast<const float*>(wsb + W.stash);
    float* part = reinterpret_cast<float*>(wsb + W.part);
    float* dxp = reinterpret_cast<float*>(wsb + W.dxp);
    float* dcb = reinterpret_cast<float*>(wsb + skew_dcb_offset(W));
    hipError_t e;
    {
        Timed t("bwd_skewed_columns");
        e = mdl::launch_skew_bwd(D, H, Ul, Uu, stash, dy_flat, dh_dirs, dA, dcb, st);
    }
    if (e != hipSuccess) return hip_fail(e, "mdl_backward_skewed: column steps");
    if (dx_canvas) {
        Timed t("zero_fill");
        e = mdl::launch_zero_outside(D, dx_canvas, C, 1, st);
        if (e != hipSuccess) return hip_fail(e, "mdl_backward_skewed: zero fill");
    }
    {
        Timed t("wgrad");
        e = mdl::launch_wgrad(D, x_canvas, x_dtype, C, H, h_dirs, dA, Wx, part, dxp, dWx, dUl, dUu, db, dx_flat,
                              dx_canvas, st);
    }
    if (e != hipSuccess) return hip_fail(e, "mdl_backward_skewed: weight and input gradients");
    return MDL_OK;
    GUARD_END
}

int mdl_dirsum_unpack(const mdl_layout* layout, const void* d_desc, const float* h_dirs, int32_t H, float* y_flat,
                      void* stream) {
    GUARD_BEGIN
    int rc = check_layer("mdl_dirsum_unpack", layout, d_desc, 1, H, MDL_F32);
    if (rc) return rc;
    if (!h_dirs || !y_flat) return fail(MDL_EINVAL, "mdl_dirsum_unpack: null tensor");
    hipError_t e;
    {
        Timed t("dirsum");
        e = mdl::launch_dirsum(make_dev(layout, d_desc), h_dirs, H, y_flat, static_cast<hipStream_t>(stream));
    }
    if (e != hipSuccess) return hip_fail(e, "mdl_dirsum_unpack");
    return MDL_OK;
    GUARD_END
}

int mdl_backward(const mdl_layout* layout, const void* d_desc, const void* x_canvas, int32_t x_dtype, int32_t C,
                 int32_t H, int32_t cell, const float* Wx, const float* Ul, const float* Uu, const float* Vl,
                 const float* Vu, const float* h_dirs, const float* dy_flat, const float* dh_dirs, float* dx_flat,
                 float* dx_canvas, float* dWx, float* dUl, float* dUu, float* db, float* dVl, float* dVu, void* ws,
                 size_t ws_bytes, void* stream) {
    GUARD_BEGIN
    int rc = check_layer("mdl_backward", layout, d_desc, C, H, x_dtype);
    if (rc) return rc;
    if ((rc = check_cell("mdl_backward", cell, Vl, Vu))) return rc;
    const bool lk = cell == MDL_CELL_LEAKY_LP;
    if (lk != (dVl != nullptr) || lk != (dVu != nullptr))
        return fail(MDL_EINVAL, "mdl_backward: dVl and dVu go with the Leaky LP cell, and only with it");
    if (!x_canvas || !Wx || !Ul || !Uu || !h_dirs || !ws) return fail(MDL_EINVAL, "mdl_backward: null tensor");
    if (!dWx || !dUl || !dUu || !db) return fail(MDL_EINVAL, "mdl_backward: null weight-gradient output");
    if ((dy_flat == nullptr) == (dh_dirs == nullptr))
        return fail(MDL_EINVAL, "mdl_backward: pass exactly one of dy_flat and dh_dirs");
    const mdl::Layout& L = L_of(layout);
    const mdl::WsLayout W = mdl::ws_layout(L.computed_cells, L.nparts(), C, H, nflags_of(L), nfflags_of(L));
    if (ws_bytes < W.total) return fail(MDL_ESIZE, "mdl_backward: workspace smaller than mdl_workspace_size");
    if (lk && !mdl::leaky_supported(H, C, L.max_diag))
        return fail(MDL_EUNSUPPORTED, "mdl_backward: the Leaky LP cell runs for H in {4, 8, 16, 32}, C <= 16 and a "
                                      "widest diagonal of at most 64 cells (32 at H = 32)");
    if (!lk && !mdl::small_bwd_supported(H, L.max_diag) && !mdl::bwd16_supported(H, L.max_diag) &&
        !mdl::chain_uses_mfma(H, L.max_diag) &&
        (int64_t)L.max_diag * H > mdl::chain_max_items())
        return fail(MDL_EUNSUPPORTED, "mdl_backward: widest diagonal x H exceeds the wavefront kernel's items");
    const bool wg2 = mdl::wgrad2_supported(C, H, x_dtype);
    if ((rc = check_extent("mdl_backward", L, C, H, x_dtype, true))) return rc;
    size_t lmax = 0;
    if ((rc = max_lds(lmax))) return rc;
    if ((lk ? mdl::leaky_bwd_lds(H, L.max_diag) : mdl::bwd_chain_lds(H, L.max_diag)) > lmax)
        return fail(MDL_EUNSUPPORTED, "mdl_backward: recurrent weights and diagonal state exceed LDS");
    if ((wg2 ? mdl::wgrad2_lds_bytes(C, H, x_dtype) : mdl::wgrad_lds_bytes(C, H)) > lmax)
        return fail(MDL_EUNSUPPORTED, "mdl_backward: weight-gradient tile exceeds LDS");
    const mdl::Dev D = make_dev(layout, d_desc);
    hipStream_t st = static_cast<hipStream_t>(stream);
    uint8_t* wsb = static_cast<uint8_t*>(ws);
    float* dA = reinterpret_cast<float*>(wsb + W.zda);
    const float* stash = reinterpret_cast<const float*>(wsb + W.stash);
    float* part = reinterpret_cast<float*>(wsb + W.part);
    float* dxp = reinterpret_cast<float*>(wsb + W.dxp);
    const bool want_dx = dx_flat != nullptr || dx_canvas != nullptr;
    hipError_t e;
    // The weight gradient overlaps the reverse wavefront when the wavefront's units leave at least half of
    // the compute units free: each unit flags itself when done, and persistent workgroups on a second
    // stream (one per free compute unit, so the wavefront's units always find room) take the weight-gradient
    // tasks (one direction of one group) from a claim queue, in the order their units finish, once those
    // units are done. The launch after the wavefront takes the rest of the queue on every compute unit while
    // they finish their last tasks; a third launch, after both, does any task given up beside the wavefront
    // for want of time. Each task is computed by the same code either way.
    Side* side = nullptr;
    int ov_wg = 0;
    const int ov_mode = g_overlap.load();
    // (the Leaky-LP cell's gate gradients have the plain cell's layout: the same tasks, once its 16-bit reverse
    // wavefront flags its units)
    if (ov_mode != 0 && wg2 && (lk ? mdl::leaky16_used(H, L.max_diag) : mdl::bwd16_supported(H, L.max_diag))) {
        if ((rc = side_of(side))) return rc;
        const int free_cu = side->ncu - 4 * L.n;
        if (2 * free_cu >= side->ncu) ov_wg = std::min(free_cu, 4 * (int)L.ngroups);
    }
    mdl::OverlapFlags F{};
    if (ov_wg > 0) {
        int32_t* fl = reinterpret_cast<int32_t*>(wsb + W.flags);
        F.done = fl;
        F.taken = fl + 4 * L.n;
        F.abandoned = F.taken + 4 * L.ngroups;
        F.queue = F.abandoned + 4 * L.ngroups;
        F.stop = F.queue + 1;
        F.nab = F.queue + 2;
        F.abq = F.queue + 3;
        if ((e = mdl::launch_fill_i32(fl, nflags_of(L), 0, st)) != hipSuccess)
            return hip_fail(e, "mdl_backward: overlap counters");
        if ((e = hipEventRecord(side->fork, st)) != hipSuccess || (e = hipStreamWaitEvent(side->s, side->fork, 0)) != hipSuccess)
            return hip_fail(e, "mdl_backward: fork to the weight-gradient stream");
    }
    {
        Timed t("bwd_wavefront");
        e = lk ? (ov_wg > 0 ? mdl::launch_bwd_leaky16(D, H, Ul, Uu, Vl, Vu, stash, dy_flat, dh_dirs, dA, F.done, st)
                            : mdl::launch_bwd_leaky(D, H, Ul, Uu, Vl, Vu, stash, dy_flat, dh_dirs, dA, st))
           : ov_wg > 0 ? mdl::launch_bwd16(D, H, Ul, Uu, stash, dy_flat, dh_dirs, dA, F.done, st)
                       : mdl::launch_bwd_chain(D, H, Ul, Uu, stash, dy_flat, dh_dirs, dA, st);
    }
    if (e != hipSuccess) return hip_fail(e, "mdl_backward: reverse wavefront");
    if (dx_canvas) {
        Timed t("zero_fill");
        e = mdl::launch_zero_outside(D, dx_canvas, C, 1, st);
        if (e != hipSuccess) return hip_fail(e, "mdl_backward: zero fill");
    }
    if (ov_wg > 0) {
        // each wait at most ~2^15 clock cycles per dependent step of the layout (several times the reverse
        // wavefront's own time per step), at least 2^26 cycles
        const long long budget = ov_mode == 2 ? 0 : std::max<long long>(1ll << 26, (long long)L.max_depth << 15);
        {
            Timed t("wgrad_overlap");
            e = mdl::launch_wgrad2_claim(D, x_canvas, x_dtype, C, H, h_dirs, dA, Wx, part, want_dx ? dxp : nullptr,
                                         F, mdl::kClaimBeside, ov_wg, budget, 0, side->s);
        }
        if (e != hipSuccess) return hip_fail(e, "mdl_backward: weight gradients beside the reverse wavefront");
        if ((e = hipEventRecord(side->join, side->s)) != hipSuccess)
            return hip_fail(e, "mdl_backward: weight-gradient stream");
        {
            Timed t("wgrad");
            e = mdl::launch_wgrad2_claim(D, x_canvas, x_dtype, C, H, h_dirs, dA, Wx, part, want_dx ? dxp : nullptr,
                                         F, mdl::kClaimDrain, 0, 0, 0, st);
            if (e == hipSuccess && (e = hipStreamWaitEvent(st, side->join, 0)) == hipSuccess)
                e = mdl::launch_wgrad2_claim(D, x_canvas, x_dtype, C, H, h_dirs, dA, Wx, part,
                                             want_dx ? dxp : nullptr, F, mdl::kClaimAbandoned, 16, 0, 0, st);
            if (e == hipSuccess) e = mdl::launch_dx_sum(D, C, dxp, dx_flat, dx_canvas, st);
            if (e == hipSuccess) e = mdl::launch_wgrad_reduce(L.ngroups, C, H, part, dWx, dUl, dUu, db, st);
        }
        if (e != hipSuccess) return hip_fail(e, "mdl_backward: weight and input gradients");
    } else {
        Timed t("wgrad");
        e = mdl::launch_wgrad(D, x_canvas, x_dtype, C, H, h_dirs, dA, Wx, part, dxp, dWx, dUl, dUu, db, dx_flat,
                              dx_canvas, st);
        if (e != hipSuccess) return hip_fail(e, "mdl_backward: weight and input gradients");
    }
    if (lk) {
        // the memory-state projections' gradients, their partials in the partial-sum buffer the weight gradients
        // above are done with ([ngroups][4][2H][3H] fits in its [nparts][4][C+1+2H][5H])
        Timed t("wgrad_mem");
        e = mdl::launch_dv_leaky(D, H, stash, dA, part, dVl, dVu, st);
        if (e != hipSuccess) return hip_fail(e, "mdl_backward: memory-state projection gradients");
    }
    return MDL_OK;
    GUARD_END
}

static int check_conv(const char* fn, const mdl_layout* lk, const void* dk, const mdl_layout* lk1, const void* dk1,
                      int32_t H, int32_t kh, int32_t kw, int32_t Cout) {
    if (!lk || !dk || !lk1 || !dk1) return fail(MDL_EINVAL, std::string(fn) + ": null layout or descriptor");
    if (H < 1 || kh < 1 || kw < 1 || Cout < 1) return fail(MDL_EINVAL, std::string(fn) + ": non-positive size");
    const mdl::Layout& A = L_of(lk);
    const mdl::Layout& B = L_of(lk1);
    if (A.n != B.n) return fail(MDL_EINVAL, std::string(fn) + ": layouts hold different example counts");
    for (int e = 0; e < A.n; ++e) {
        const int h = A.real[4 * e + 2], w = A.real[4 * e + 3];
        if (B.real[4 * e + 2] != (h + kh - 1) / kh || B.real[4 * e + 3] != (w + kw - 1) / kw)
            return fail(MDL_EINVAL, std::string(fn) + ": level-(k+1) example sizes are not ceil(h/kh) x ceil(w/kw)");
    }
    return MDL_OK;
}

int mdl_blockconv_forward(const mdl_layout* lk, const void* d_desc_k, const mdl_layout* lk1, const void* d_desc_k1,
                          const float* h_dirs_k, int32_t H, int32_t kh, int32_t kw, const float* Wc, const float* bc,
                          int32_t Cout, float* x_canvas_k1, void* stream) {
    GUARD_BEGIN
    int rc = check_conv("mdl_blockconv_forward", lk, d_desc_k, lk1, d_desc_k1, H, kh, kw, Cout);
    if (rc) return rc;
    if (!h_dirs_k || !Wc || !bc || !x_canvas_k1) return fail(MDL_EINVAL, "mdl_blockconv_forward: null tensor");
    size_t lmax = 0;
    if ((rc = max_lds(lmax))) return rc;
    if (mdl::conv_fwd_lds(H, kh, kw, Cout) > lmax)
        return fail(MDL_EUNSUPPORTED, "mdl_blockconv_forward: weights and block tile exceed LDS");
    hipError_t e;
    {
        Timed t("conv_fwd");
        e = mdl::launch_conv_fwd(make_dev(lk, d_desc_k), make_dev(lk1, d_desc_k1), h_dirs_k, H, kh, kw, Wc, bc, Cout,
                                 x_canvas_k1, static_cast<hipStream_t>(stream));
    }
    if (e != hipSuccess) return hip_fail(e, "mdl_blockconv_forward");
    return MDL_OK;
    GUARD_END
}

int mdl_blockconv_workspace_size(const mdl_layout* lk1, int32_t H, int32_t kh, int32_t kw, int32_t Cout,
                                 size_t* bytes) {
    if (!lk1 || !bytes) return fail(MDL_EINVAL, "mdl_blockconv_workspace_size: null argument");
    if (H < 1 || kh < 1 || kw < 1 || Cout < 1) return fail(MDL_EINVAL, "mdl_blockconv_workspace_size: non-positive size");
    const mdl::Layout& B = L_of(lk1);
    mdl::Dev D{};
    D.N = B.real_pixels;
    D.Hc = B.Hc;
    D.Wc = B.Wc;
    const int64_t K = 4 * (int64_t)H * kh * kw;
    *bytes = sizeof(float) * (size_t)mdl::conv_nchunks(D) * (size_t)(Cout * (K + 1));
    return MDL_OK;
}

static int conv_bwd(const char* fn, const mdl_layout* lk, const void* d_desc_k, const mdl_layout* lk1,
                    const void* d_desc_k1, const float* h_dirs_k, int32_t H, int32_t kh, int32_t kw, const float* Wc,
                    int32_t Cout, const float* dx_canvas_k1, float* dh_dirs_k, float* dWc, float* dbc, void* ws,
                    size_t ws_bytes, bool fixed_scratch, void* stream) {
    int rc = check_conv(fn, lk, d_desc_k, lk1, d_desc_k1, H, kh, kw, Cout);
    if (rc) return rc;
    if (!h_dirs_k || !Wc || !dx_canvas_k1 || !dh_dirs_k || !dWc || !dbc || !ws)
        return fail(MDL_EINVAL, std::string(fn) + ": null tensor");
    const int64_t K = 4 * (int64_t)H * kh * kw;
    if (Cout * (K + 1) > 16 * 512) return fail(MDL_EUNSUPPORTED, std::string(fn) + ": Cout*(4*H*kh*kw+1) above 8192");
    size_t need = 0;
    mdl_blockconv_workspace_size(lk1, H, kh, kw, Cout, &need);
    if (ws_bytes < need) {
        if (fixed_scratch)
            return fail(MDL_ESIZE, std::string(fn) + ": the weight-gradient partials need " + std::to_string(need) +
                                       " bytes, above the library's fixed scratch of " + std::to_string(ws_bytes));
        return fail(MDL_ESIZE, std::string(fn) + ": workspace too small");
    }
    size_t lmax = 0;
    if ((rc = max_lds(lmax))) return rc;
    if (mdl::conv_wgrad_lds(H, kh, kw, Cout) > lmax || mdl::conv_data_lds(H, kh, kw, Cout) > lmax)
        return fail(MDL_EUNSUPPORTED, std::string(fn) + ": weight-gradient tile or weights exceed LDS");
    hipError_t e;
    {
        Timed t("conv_bwd");
        e = mdl::launch_conv_bwd(make_dev(lk, d_desc_k), make_dev(lk1, d_desc_k1), h_dirs_k, H, kh, kw, Wc, Cout,
                                 dx_canvas_k1, dh_dirs_k, dWc, dbc, static_cast<float*>(ws),
                                 static_cast<hipStream_t>(stream));
    }
    if (e != hipSuccess) return hip_fail(e, fn);
    return MDL_OK;
}

int mdl_blockconv_backward(const mdl_layout* lk, const void* d_desc_k, const mdl_layout* lk1, const void* d_desc_k1,
                           const float* h_dirs_k, int32_t H, int32_t kh, int32_t kw, const float* Wc, int32_t Cout,
                           const float* dx_canvas_k1, float* dh_dirs_k, float* dWc, float* dbc, void* ws,
                           size_t ws_bytes, void* stream) {
    GUARD_BEGIN
    return conv_bwd("mdl_blockconv_backward", lk, d_desc_k, lk1, d_desc_k1, h_dirs_k, H, kh, kw, Wc, Cout,
                    dx_canvas_k1, dh_dirs_k, dWc, dbc, ws, ws_bytes, false, stream);
    GUARD_END
}

int mdl_blockconv_backward_noalloc(const mdl_layout* lk, const void* d_desc_k, const mdl_layout* lk1,
                                   const void* d_desc_k1, const float* h_dirs_k, int32_t H, int32_t kh, int32_t kw,
                                   const float* Wc, int32_t Cout, const float* dx_canvas_k1, float* dh_dirs_k,
                                   float* dWc, float* dbc, void* stream) {
    GUARD_BEGIN
    const char* fn = "mdl_blockconv_backward_noalloc";
    int rc = check_conv(fn, lk, d_desc_k, lk1, d_desc_k1, H, kh, kw, Cout);
    if (rc) return rc;
    void* ws = nullptr;
    size_t cap = 0;
    const hipError_t e = mdl::conv_scratch(&ws, &cap);
    if (e != hipSuccess) return hip_fail(e, "mdl_blockconv_backward_noalloc: scratch address");
    return conv_bwd(fn, lk, d_desc_k, lk1, d_desc_k1, h_dirs_k, H, kh, kw, Wc, Cout, dx_canvas_k1, dh_dirs_k, dWc,
                    dbc, ws, cap, true, stream);
    GUARD_END
}

static int ctc_tmax(const mdl::Layout& L) {
    int t = 0;
    for (int e = 0; e < L.n; ++e) t = std::max(t, L.real[4 * e + 3]);
    return t;
}

static int check_ctc(const char* fn, const mdl_layout* layout, int32_t H, int32_t K, int32_t max_label) {
    if (!layout) return fail(MDL_EINVAL, std::string(fn) + ": null layout");
    if (H < 1 || K < 2 || max_label < 0)
        return fail(MDL_EINVAL, std::string(fn) + ": need H >= 1, K >= 2 and max_label >= 0");
    if (H > 1024 || K > 4096 || max_label > 65535)
        return fail(MDL_EUNSUPPORTED, std::string(fn) + ": H above 1024, K above 4096 or max_label above 65535");
    const int64_t T = ctc_tmax(L_of(layout));
    const int64_t S = 2 * (int64_t)max_label + 1;
    if (T * std::max<int64_t>(std::max<int64_t>(H, K), S) >= (int64_t(1) << 31))
        return fail(MDL_EOVERFLOW, std::string(fn) + ": frames times classes, hidden units or label states reach 2^31");
    return MDL_OK;
}

int mdl_ctc_workspace_size(const mdl_layout* layout, int32_t H, int32_t K, int32_t max_label, size_t* bytes) {
    GUARD_BEGIN
    if (!bytes) return fail(MDL_EINVAL, "mdl_ctc_workspace_size: null argument");
    int rc = check_ctc("mdl_ctc_workspace_size", layout, H, K, max_label);
    if (rc) return rc;
    const mdl::Layout& L = L_of(layout);
    *bytes = sizeof(float) * (size_t)mdl::ctc_ws(L.n, ctc_tmax(L), H, K, max_label).total;
    return MDL_OK;
    GUARD_END
}

int mdl_ctc_head(const mdl_layout* layout, const void* d_desc, const float* y_flat, int32_t H, const float* Wfc,
                 const float* bfc, int32_t K, const int32_t* labels, const int32_t* label_off, int64_t n_labels,
                 int32_t max_label, float* loss, float* dy_flat, float* dWfc, float* dbfc, void* ws,
                 size_t ws_bytes, void* stream) {
    GUARD_BEGIN
    int rc = check_ctc("mdl_ctc_head", layout, H, K, max_label);
    if (rc) return rc;
    if (!d_desc || !y_flat || !Wfc || !bfc || !label_off || !loss || !ws)
        return fail(MDL_EINVAL, "mdl_ctc_head: null tensor");
    if (n_labels < 0 || (n_labels > 0 && !labels)) return fail(MDL_EINVAL, "mdl_ctc_head: bad label array");
    if ((dWfc == nullptr) != (dbfc == nullptr))
        return fail(MDL_EINVAL, "mdl_ctc_head: give both dWfc and dbfc, or neither");
    const mdl::Layout& L = L_of(layout);
    const int Tmax = ctc_tmax(L);
    const size_t need = sizeof(float) * (size_t)mdl::ctc_ws(L.n, Tmax, H, K, max_label).total;
    if (ws_bytes < need) return fail(MDL_ESIZE, "mdl_ctc_head: workspace smaller than mdl_ctc_workspace_size");
    size_t lds = 0;
    rc = max_lds(lds);
    if (rc) return rc;
    hipError_t e;
    {
        Timed t("ctc_head");
        e = mdl::launch_ctc_head(make_dev(layout, d_desc), y_flat, H, Wfc, bfc, K, labels, label_off, n_labels,
                                 max_label, Tmax, static_cast<float*>(ws), loss, dy_flat, dWfc, dbfc, lds,
                                 static_cast<hipStream_t>(stream));
    }
    if (e != hipSuccess) return hip_fail(e, "mdl_ctc_head");
    return MDL_OK;
    GUARD_END
}

int mdl_set_wgrad_overlap(int32_t mode) {
    if (mode < 0 || mode > 2) return fail(MDL_EINVAL, "mdl_set_wgrad_overlap: mode must be 0, 1 or 2");
    g_overlap.store(mode);
    return MDL_OK;
}

int mdl_timing(int32_t enable) {
    std::lock_guard<std::mutex> lk(g_tmu);
    g_timing = enable != 0;
    return MDL_OK;
}

int mdl_timing_only(const char* group) {
    if (group && std::strlen(group) >= 32) return fail(MDL_EINVAL, "mdl_timing_only: group name too long");
    std::lock_guard<std::mutex> lk(g_tmu);
    g_timing_only = group ? group : "";
    return MDL_OK;
}

int mdl_timing_report(int32_t max, char* names, double* total_ms, int64_t* launches, int32_t* count) {
    GUARD_BEGIN
    if (max < 0 || !count || (max > 0 && (!names || !total_ms || !launches)))
        return fail(MDL_EINVAL, "mdl_timing_report: bad arguments");
    std::lock_guard<std::mutex> lk(g_tmu);
    std::map<std::string, std::pair<double, int64_t>> acc;
    std::vector<std::string> order;
    int rc = MDL_OK;
    for (auto& t : g_tlog) {
        float ms = 0.f;
        hipError_t e = hipEventSynchronize(t.ev.back());
        if (e == hipSuccess) e = hipEventElapsedTime(&ms, t.ev.front(), t.ev.back());
        if (e != hipSuccess && rc == MDL_OK) rc = hip_fail(e, "mdl_timing_report");
        if (!acc.count(t.name)) order.push_back(t.name);
        acc[t.name].first += ms;
        acc[t.name].second += 1;
        for (hipEvent_t ev : t.ev) g_event_pool.push_back(ev);
    }
    g_tlog.clear();
    int k = 0;
    for (const auto& nm : order) {
        if (k >= max) break;
        std::memset(names + 32 * k, 0, 32);
        std::strncpy(names + 32 * k, nm.c_str(), 31);
        total_ms[k] = acc[nm].first;
        launches[k] = acc[nm].second;
        ++k;
    }
    *count = k;
    return rc;
    GUARD_END
}

const char* mdl_last_error(void) { return g_err.c_str(); }

}  // extern "C"
