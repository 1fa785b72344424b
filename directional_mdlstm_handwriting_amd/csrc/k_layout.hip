// k_layout.hip — canvas maps, scatter onto the canvas, direction sum + un-packing.
//
// "No Padding Please", §V: the binary mask marks example pixels (here with the
// example id) so that state from padding or separator predecessors is
// blocked; §V-A: un-packing cuts each example's activations out of the canvas
// by its original index and size. All of these are HBM-bound copies: one
// thread per output element, consecutive threads on consecutive addresses.
#include "kernels.h"
#include "devmath.h"

namespace mdl {

namespace {

constexpr int TPB = 256;
// the direction sums: threads per workgroup (k_dirsum4 is launched with TPB of them) and elements per thread
// whose loads are in flight together
constexpr int kSumThreads = TPB;
constexpr int kSumBatch = 4;

inline unsigned grid_for(int64_t n, int tpb = TPB, int64_t cap = 1 << 20) {
    int64_t g = (n + tpb - 1) / tpb;
    if (g < 1) g = 1;
    return (unsigned)(g < cap ? g : cap);
}

__global__ void k_fill_eid(int32_t* __restrict__ eid, int64_t P) {
    for (int64_t p = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; p < P; p += (int64_t)gridDim.x * blockDim.x)
        eid[p] = -1;
}

__global__ void k_fill_i32(int32_t* __restrict__ p, int64_t n, int32_t v) {
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
        p[i] = v;
}

// blockIdx.y = example; paints its computed region
__global__ void k_paint_eid(Dev D) {
    const int e = blockIdx.y;
    const int y0 = D.rect[4 * e], x0 = D.rect[4 * e + 1], h = D.rect[4 * e + 2], w = D.rect[4 * e + 3];
    const int64_t cells = (int64_t)h * w;
    for (int64_t q = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; q < cells; q += (int64_t)gridDim.x * blockDim.x) {
        const int ly = (int)(q / w), lx = (int)(q % w);
        D.eid[(int64_t)(y0 + ly) * D.Wc + x0 + lx] = e;
    }
}

__global__ void k_border(Dev D) {
    const int64_t P = (int64_t)D.Hc * D.Wc;
    for (int64_t p = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; p < P; p += (int64_t)gridDim.x * blockDim.x) {
        const int y = (int)(p / D.Wc), x = (int)(p % D.Wc);
        const int e = D.eid[p];
        uint8_t bits = 0;
        if (e >= 0) {
            if (x > 0 && D.eid[p - 1] == e) bits |= 1;
            if (x + 1 < D.Wc && D.eid[p + 1] == e) bits |= 2;
            if (y > 0 && D.eid[p - D.Wc] == e) bits |= 4;
            if (y + 1 < D.Hc && D.eid[p + D.Wc] == e) bits |= 8;
        }
        D.border[p] = bits;
    }
}

// One thread per canvas element (pixel, channel): copy from the example's flat
// tensor inside its real rectangle, zero elsewhere.
template <typename T>
__global__ void k_scatter(Dev D, const T* __restrict__ xf, int C, T* __restrict__ xc) {
    const int64_t E = (int64_t)D.Hc * D.Wc * C;
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < E; i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t p = i / C;
        const int c = (int)(i % C);
        const int e = D.eid[p];
        T v = T(0);
        if (e >= 0) {
            const int y = (int)(p / D.Wc), x = (int)(p % D.Wc);
            const int ry = y - D.real[4 * e], rx = x - D.real[4 * e + 1];
            const int rh = D.real[4 * e + 2], rw = D.real[4 * e + 3];
            if (ry < rh && rx < rw) v = xf[(D.flat_off[e] + (int64_t)ry * rw + rx) * C + c];
        }
        xc[i] = v;
    }
}

// Whole-pixel forms of the copies above, for the common shapes: one thread per canvas pixel (scatter, a pixel's
// C channels as one 8- or 16-byte vector V) or per 16-byte group of a pixel's values (zero fill, direction sum),
// canvas rows on blockIdx.y (a grid-stride loop past 65535 rows), 32-bit index arithmetic inside a row or an
// example. Same results as the element forms, bit for bit.
template <typename V>
__global__ void k_scatter_px(Dev D, const V* __restrict__ xf, V* __restrict__ xc) {
    const int x = blockIdx.x * blockDim.x + threadIdx.x;
    if (x >= D.Wc) return;
    for (int y = blockIdx.y; y < D.Hc; y += gridDim.y) {
        const int64_t p = (int64_t)y * D.Wc + x;
        const int e = D.eid[p];
        V v = {};
        if (e >= 0) {
            const int ry = y - D.real[4 * e], rx = x - D.real[4 * e + 1];
            const int rh = D.real[4 * e + 2], rw = D.real[4 * e + 3];
            if (ry < rh && rx < rw) v = xf[D.flat_off[e] + (int64_t)ry * rw + rx];
        }
        xc[p] = v;
    }
}

// K4 = K / 4 float4 groups per pixel; plane4 = Hc * Wc * K4
__global__ void k_zero_outside4(Dev D, f32x4* __restrict__ buf, int K4, int planes, int64_t plane4) {
    const int q = blockIdx.x * blockDim.x + threadIdx.x;  // float4 group within the canvas row
    if (q >= D.Wc * K4) return;
    const int x = q / K4;
    for (int y = blockIdx.y; y < D.Hc; y += gridDim.y) {
        if (D.eid[(int64_t)y * D.Wc + x] >= 0) continue;
        const int64_t i = (int64_t)y * D.Wc * K4 + q;
        for (int pl = 0; pl < planes; ++pl) buf[pl * plane4 + i] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
}

// blockIdx.y = example; H4 = H / 4
__global__ void k_dirsum4(Dev D, const f32x4* __restrict__ hd, int H4, f32x4* __restrict__ y) {
    const int e = blockIdx.y;
    const int y0 = D.real[4 * e], x0 = D.real[4 * e + 1], rh = D.real[4 * e + 2], rw = D.real[4 * e + 3];
    const int cnt = rh * rw * H4;
    const int64_t plane = (int64_t)D.Hc * D.Wc * H4;
    f32x4* out = y + D.flat_off[e] * H4;
    // kSumBatch elements per thread at a time, all their loads issued before the first sum
    const int stride = (int)gridDim.x * kSumThreads;
    for (int q0 = blockIdx.x * kSumThreads + threadIdx.x; q0 < cnt; q0 += kSumBatch * stride) {
        f32x4 v[kSumBatch][4];
#pragma unroll
        for (int j = 0; j < kSumBatch; ++j) {
            const int q = q0 + j * stride;
            const int pix = q / H4, k = q - pix * H4;
            const int ly = pix / rw, lx = pix - ly * rw;
            const int64_t src = ((int64_t)(y0 + ly) * D.Wc + x0 + lx) * H4 + k;
#pragma unroll
            for (int d = 0; d < 4; ++d) v[j][d] = q < cnt ? hd[src + d * plane] : f32x4{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int j = 0; j < kSumBatch; ++j)
            if (q0 + j * stride < cnt) out[q0 + j * stride] = ((v[j][0] + v[j][1]) + v[j][2]) + v[j][3];
    }
}

// ---- the direction sum beside the forward wavefront ----


// chunk i of the layout's direction-sum chunks (example e, real pixels [p0, p1) row-major): y of those pixels,
// the directions added in order as in k_dirsum4
__device__ __forceinline__ void dsum_chunk(const Dev& D, const f32x4* __restrict__ hd, int H4,
                                           f32x4* __restrict__ y, int i) {
    const int e = D.dsum[3 * i], p0 = D.dsum[3 * i + 1], p1 = D.dsum[3 * i + 2];
    const int y0 = D.real[4 * e], x0 = D.real[4 * e + 1], rw = D.real[4 * e + 3];
    const int64_t plane = (int64_t)D.Hc * D.Wc * H4;
    f32x4* out = y + D.flat_off[e] * H4;
    const int n = (p1 - p0) * H4;
    // kSumBatch elements per thread at a time, all their loads issued before the first sum
    for (int q0 = threadIdx.x; q0 < n; q0 += kSumBatch * kSumThreads) {
        f32x4 v[kSumBatch][4];
        int64_t dst[kSumBatch];
#pragma unroll
        for (int j = 0; j < kSumBatch; ++j) {
            const int q = q0 + j * kSumThreads;
            const int pq = q / H4, k = q - pq * H4;
            const int pix = p0 + pq;
            const int ly = pix / rw, lx = pix - ly * rw;
            const int64_t src = ((int64_t)(y0 + ly) * D.Wc + x0 + lx) * H4 + k;
            dst[j] = q < n ? (int64_t)pix * H4 + k : -1;
#pragma unroll
            for (int d = 0; d < 4; ++d) v[j][d] = q < n ? hd[src + d * plane] : f32x4{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int j = 0; j < kSumBatch; ++j)
            if (dst[j] >= 0) out[dst[j]] = ((v[j][0] + v[j][1]) + v[j][2]) + v[j][3];
    }
}

// Thread 0 of a workgroup beside the forward takes its next chunk: the next queue position (unless the stop
// flag is set) whose taken flag it is first to set, then waits until the four forward units of the chunk's
// example are flagged (polled without ordering, one acquire fence at the end; bounded by `budget` shader
// clocks, past which the position goes on the abandoned list and the stop flag ends claiming). For the
// abandoned list, the next entry. Returns the position, or -1 once there is none to take.
__device__ int claim_chunk(const Dev& D, const OverlapFlags& F, int mode, long long budget) {
    if (mode == kClaimAbandoned) {
        const int i = __hip_atomic_fetch_add(F.abq, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        return i < __hip_atomic_load(F.nab, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ? F.abandoned[i] : -1;
    }
    int qi;
    do {
        if (__hip_atomic_load(F.stop, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0) return -1;
        qi = __hip_atomic_fetch_add(F.queue, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (qi >= D.nsum) return -1;
    } while (__hip_atomic_exchange(F.taken + qi, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0);
    const int e = D.dsum[3 * qi];
    const unsigned long long t0 = __builtin_amdgcn_s_memtime();
    for (int d = 0; d < 4; ++d) {
        while (__hip_atomic_load(F.done + 4 * e + d, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 0) {
            if ((long long)(__builtin_amdgcn_s_memtime() - t0) > budget) {
                const int k = __hip_atomic_fetch_add(F.nab, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                F.abandoned[k] = qi;
                __hip_atomic_store(F.stop, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                return -1;
            }
            __builtin_amdgcn_s_sleep(16);
        }
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    return qi;
}

// Chunks claimed one after another until none is left: persistent workgroups beside the forward, or the
// abandoned list after the join.
__global__ __launch_bounds__(kSumThreads) void k_dsum_claim(Dev D, const f32x4* __restrict__ hd, int H4,
                                                            f32x4* __restrict__ y, OverlapFlags F, int mode,
                                                            long long budget) {
    __shared__ int s_pos;
    // one thread-0 region per iteration, barriers closing every iteration (as in the weight gradients' claim)
    for (;;) {
        if (threadIdx.x == 0) s_pos = claim_chunk(D, F, mode, budget);
        __syncthreads();
        const int pos = s_pos;
        __syncthreads();
        if (pos < 0) break;
        dsum_chunk(D, hd, H4, y, pos);
        __syncthreads();
    }
}

// After the forward on its stream: workgroup b takes queue position b unless a workgroup beside the forward
// has taken it (every unit is complete, so nothing is waited for).
__global__ __launch_bounds__(kSumThreads) void k_dsum_drain(Dev D, const f32x4* __restrict__ hd, int H4,
                                                            f32x4* __restrict__ y, OverlapFlags F) {
    __shared__ int s_taken;
    if (threadIdx.x == 0)
        s_taken = __hip_atomic_exchange(F.taken + blockIdx.x, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    if (s_taken != 0) return;
    dsum_chunk(D, hd, H4, y, blockIdx.x);
}

// blockIdx.y = example: y_flat[e][r][c][k] = sum_d h_dirs[d][y0+r][x0+c][k], d = 0..3 in order
__global__ void k_dirsum(Dev D, const float* __restrict__ hd, int H, float* __restrict__ y) {
    const int e = blockIdx.y;
    const int y0 = D.real[4 * e], x0 = D.real[4 * e + 1], rh = D.real[4 * e + 2], rw = D.real[4 * e + 3];
    const int64_t cnt = (int64_t)rh * rw * H;
    const int64_t plane = (int64_t)D.Hc * D.Wc * H;
    float* out = y + D.flat_off[e] * H;
    for (int64_t q = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; q < cnt; q += (int64_t)gridDim.x * blockDim.x) {
        const int64_t pix = q / H;
        const int k = (int)(q % H);
        const int ly = (int)(pix / rw), lx = (int)(pix % rw);
        const int64_t src = ((int64_t)(y0 + ly) * D.Wc + x0 + lx) * H + k;
        float s = hd[src];
        s += hd[src + plane];
        s += hd[src + 2 * plane];
        s += hd[src + 3 * plane];
        out[q] = s;
    }
}

// zero `planes` planes of [Hc*Wc][K] floats at every pixel outside all computed regions
__global__ void k_zero_outside(Dev D, float* __restrict__ buf, int K, int planes) {
    const int64_t P = (int64_t)D.Hc * D.Wc;
    const int64_t E = P * K;
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < E; i += (int64_t)gridDim.x * blockDim.x) {
        if (D.eid[i / K] >= 0) continue;
        for (int pl = 0; pl < planes; ++pl) buf[pl * E + i] = 0.f;
    }
}

}  // namespace

namespace {
bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }
unsigned rows_grid(int Hc) { return (unsigned)(Hc < 65535 ? Hc : 65535); }
}  // namespace

hipError_t launch_zero_outside(const Dev& D, float* buf, int K, int planes, hipStream_t st) {
    const int64_t E = (int64_t)D.Hc * D.Wc * K;
    if (K % 4 == 0 && aligned(buf, 16) && (int64_t)D.Wc * (K / 4) < (int64_t(1) << 31)) {
        const int K4 = K / 4;
        launch(k_zero_outside4, dim3((unsigned)(((int64_t)D.Wc * K4 + TPB - 1) / TPB), rows_grid(D.Hc)), dim3(TPB), 0,
               st, D, reinterpret_cast<f32x4*>(buf), K4, planes, E / 4);
    } else {
        launch(k_zero_outside, dim3(grid_for(E)), dim3(TPB), 0, st, D, buf, K, planes);
    }
    return hipGetLastError();
}

hipError_t launch_fill_i32(int32_t* p, int64_t n, int32_t v, hipStream_t st) {
    launch(k_fill_i32, dim3(grid_for(n)), dim3(TPB), 0, st, p, n, v);
    return hipGetLastError();
}

hipError_t launch_build_maps(const Dev& D, hipStream_t st) {
    const int64_t P = (int64_t)D.Hc * D.Wc;
    launch(k_fill_eid, dim3(grid_for(P)), dim3(TPB), 0, st, D.eid, P);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    launch(k_paint_eid, dim3(64, D.n), dim3(TPB), 0, st, D);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
    launch(k_border, dim3(grid_for(P)), dim3(TPB), 0, st, D);
    return hipGetLastError();
}

hipError_t launch_scatter(const Dev& D, const void* x_flat, int C, int dtype, void* x_canvas, hipStream_t st) {
    const int64_t E = (int64_t)D.Hc * D.Wc * C;
    const int pixel_bytes = C * (dtype == 0 ? 4 : 2);
    const dim3 pgrid((unsigned)((D.Wc + TPB - 1) / TPB), rows_grid(D.Hc));
    if (pixel_bytes == 16 && aligned(x_flat, 16) && aligned(x_canvas, 16))
        launch(k_scatter_px<u32x4>, pgrid, dim3(TPB), 0, st, D, (const u32x4*)x_flat, (u32x4*)x_canvas);
    else if (pixel_bytes == 8 && aligned(x_flat, 8) && aligned(x_canvas, 8))
        launch(k_scatter_px<u32x2>, pgrid, dim3(TPB), 0, st, D, (const u32x2*)x_flat, (u32x2*)x_canvas);
    else if (dtype == 0)
        launch(k_scatter<float>, dim3(grid_for(E)), dim3(TPB), 0, st, D,
               (const float*)x_flat, C, (float*)x_canvas);
    else
        launch(k_scatter<uint16_t>, dim3(grid_for(E)), dim3(TPB), 0, st, D,
               (const uint16_t*)x_flat, C, (uint16_t*)x_canvas);
    return hipGetLastError();
}

bool dirsum_chunked_supported(const Dev& D, const float* h_dirs, int H, const float* y_flat) {
    return H % 4 == 0 && aligned(h_dirs, 16) && aligned(y_flat, 16) && D.N * (H / 4) < (int64_t(1) << 31) &&
           (int64_t)kSumChunk * (H / 4) < (int64_t(1) << 31) && D.nsum > 0;
}

hipError_t launch_dirsum_claim(const Dev& D, const float* h_dirs, int H, float* y_flat, const OverlapFlags& F,
                               WgClaim mode, int workgroups, long long budget, size_t lds_hold, hipStream_t st) {
    if (!dirsum_chunked_supported(D, h_dirs, H, y_flat) || budget < 0) return hipErrorInvalidValue;
    const f32x4* hd = reinterpret_cast<const f32x4*>(h_dirs);
    f32x4* y = reinterpret_cast<f32x4*>(y_flat);
    if (mode == kClaimDrain)
        launch(k_dsum_drain, dim3((unsigned)D.nsum), dim3(kSumThreads), 0, st, D, hd, H / 4, y, F);
    else if (workgroups < 1)
        return hipErrorInvalidValue;
    else
        launch(k_dsum_claim, dim3((unsigned)workgroups), dim3(kSumThreads), mode == kClaimBeside ? lds_hold : 0, st, D,
               hd, H / 4, y, F, (int)mode, budget);
    return hipGetLastError();
}

hipError_t launch_dirsum(const Dev& D, const float* h_dirs, int H, float* y_flat, hipStream_t st) {
    if (H % 4 == 0 && aligned(h_dirs, 16) && aligned(y_flat, 16) && D.N * (H / 4) < (int64_t(1) << 31))
        launch(k_dirsum4, dim3(64, D.n), dim3(TPB), 0, st, D, reinterpret_cast<const f32x4*>(h_dirs), H / 4,
               reinterpret_cast<f32x4*>(y_flat));
    else
        launch(k_dirsum, dim3(64, D.n), dim3(TPB), 0, st, D, h_dirs, H, y_flat);
    return hipGetLastError();
}

}  // namespace mdl
