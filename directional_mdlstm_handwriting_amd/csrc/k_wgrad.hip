// k_wgrad.hip — weight and input gradients after the reverse wavefront.
//
// RETURNN §4.2: after the recurrent part is back-propagated through time, the
// gradients with respect to the weights and the inputs are matrix products
// over the whole batch. For direction d, with A-row r(p) = [x(p), 1, h_left(p),
// h_up(p)] (predecessors outside the example read as zero) and gate gradient
// da(p):
//     [dWx; db; dUl; dUu][d] = sum over computed cells p of r(p)^T da(p)
//     dx(p) = sum_d da_d(p) Wx[d]^T
// The sum over cells is a fixed-order two-stage reduction: chunks of
// WGRAD_CHUNK consecutive stash cells give partial sums (stage 1), which are
// added chunk by chunk in order (stage 2). No atomics, so results are
// bit-reproducible.
#include "kernels.h"

namespace mdl {

WsLayout ws_layout(int64_t T, int C, int H) {
    auto al = [](size_t v) { return (v + 255) & ~size_t(255); };
    WsLayout w;
    const int G = 5 * H;
    const int R = C + 1 + 2 * H;
    w.nchunks = (T + WGRAD_CHUNK - 1) / WGRAD_CHUNK;
    size_t p = 0;
    w.stash = p; p = al(p + sizeof(float) * 4 * (size_t)T * 6 * H);
    w.zda = p;   p = al(p + sizeof(float) * 4 * (size_t)T * G);
    w.part = p;  p = al(p + sizeof(float) * 4 * (size_t)w.nchunks * R * G);
    w.total = p;
    return w;
}

namespace {

constexpr int WG_THREADS = 1024;
constexpr int MAXE = 32;   // output entries per thread
constexpr int TILE = 32;   // cells staged in LDS at a time

template <typename XT> __device__ inline float to_f32(XT v);
template <> __device__ inline float to_f32<float>(float v) { return v; }
template <> __device__ inline float to_f32<uint16_t>(uint16_t v) { return __uint_as_float(((uint32_t)v) << 16); }

// grid (nchunks, 4): partial sums of r(p)^T da(p) over one chunk of direction d's cells
template <typename XT>
__global__ __launch_bounds__(WG_THREADS) void k_wgrad_partial(Dev D, const XT* __restrict__ xc, int C, int H,
                                                              const float* __restrict__ hdirs,
                                                              const float* __restrict__ dA,
                                                              float* __restrict__ part, int64_t nchunks) {
    const int d = blockIdx.y;
    const int64_t g0 = (int64_t)blockIdx.x * WGRAD_CHUNK;
    const int64_t g1 = g0 + WGRAD_CHUNK < D.T ? g0 + WGRAD_CHUNK : D.T;
    const int G = 5 * H, R = C + 1 + 2 * H, E = R * G;
    const bool fy = (d & 2) != 0, fx = (d & 1) != 0;
    extern __shared__ float lds[];
    float* arow = lds;                 // [TILE][R]
    float* drow = arow + TILE * R;     // [TILE][G]
    __shared__ int64_t cpix[TILE];     // canvas pixel of the cell
    __shared__ int cflag[TILE];        // bit 0: left predecessor valid, bit 1: upper, bit 2: cell exists
    const float* hd = hdirs + (int64_t)d * D.Hc * D.Wc * H;
    const float* dAd = dA + (int64_t)d * D.T * G;
    const int tid = threadIdx.x, nthr = blockDim.x;
    // thread -> one gate column and a contiguous run of A-rows of the output block
    const int tpc = nthr / G;                      // threads per column (>= 1)
    const int col = tid % G, grp = tid / G;
    const int rpt = (R + tpc - 1) / tpc;           // rows per thread (<= MAXE, checked by the host)
    const int r0 = grp * rpt;
    const bool active = grp < tpc && r0 < R;
    const int nrow = active ? (R - r0 < rpt ? R - r0 : rpt) : 0;
    float acc[MAXE];
#pragma unroll
    for (int i = 0; i < MAXE; ++i) acc[i] = 0.f;

    for (int64_t t0 = g0; t0 < g1; t0 += TILE) {
        if (tid < TILE) {
            const int64_t g = t0 + tid;
            int flag = 0;
            int64_t pix = 0;
            if (g < g1) {
                const int e = find_example(D.cell_off, D.n, g);
                const int h = D.rect[4 * e + 2], w = D.rect[4 * e + 3];
                int s, a;
                dg_decode(h, w, g - D.cell_off[e], s, a);
                const int b = s - a;
                const Flip F{D.rect[4 * e], D.rect[4 * e + 1], h, w, fy, fx};
                pix = (int64_t)F.y(a) * D.Wc + F.x(b);
                flag = 4 | (b > 0 ? 1 : 0) | (a > 0 ? 2 : 0);
            }
            cpix[tid] = pix;
            cflag[tid] = flag;
        }
        __syncthreads();
        const int sxs = fx ? -1 : 1;             // column step of the scan
        const int64_t sys = fy ? -D.Wc : D.Wc;   // row step of the scan, in pixels
        for (int idx = tid; idx < TILE * R; idx += nthr) {
            const int c = idx / R, r = idx - (idx / R) * R;
            const int f = cflag[c];
            float v = 0.f;
            if (f & 4) {
                const int64_t p = cpix[c];
                if (r < C) v = to_f32<XT>(xc[p * C + r]);
                else if (r == C) v = 1.f;
                else if (r < C + 1 + H) { if (f & 1) v = hd[(p - sxs) * H + (r - C - 1)]; }
                else { if (f & 2) v = hd[(p - sys) * H + (r - C - 1 - H)]; }
            }
            arow[idx] = v;
        }
        for (int idx = tid; idx < TILE * G; idx += nthr) {
            const int c = idx / G;
            const int64_t g = t0 + c;
            drow[idx] = g < g1 ? dAd[g * G + (idx - c * G)] : 0.f;
        }
        __syncthreads();
        if (active) {
            for (int c = 0; c < TILE; ++c) {
                const float dv = drow[c * G + col];
                const float* ar = arow + c * R + r0;
#pragma unroll
                for (int i = 0; i < MAXE; ++i)
                    if (i < nrow) acc[i] += ar[i] * dv;
            }
        }
        __syncthreads();
    }
    float* out = part + ((int64_t)d * nchunks + blockIdx.x) * E;
    if (active) {
#pragma unroll
        for (int i = 0; i < MAXE; ++i)
            if (i < nrow) out[(int64_t)(r0 + i) * G + col] = acc[i];
    }
}

// one thread per (direction, entry): chunks added in order, then routed to dWx / db / dUl / dUu
__global__ void k_wgrad_reduce(const float* __restrict__ part, int64_t nchunks, int C, int H, float* __restrict__ dWx,
                               float* __restrict__ dUl, float* __restrict__ dUu, float* __restrict__ db) {
    const int G = 5 * H, R = C + 1 + 2 * H, E = R * G;
    const int64_t id = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
    if (id >= 4 * (int64_t)E) return;
    const int d = (int)(id / E), ent = (int)(id % E);
    const float* p = part + (int64_t)d * nchunks * E + ent;
    float s = 0.f;
    for (int64_t c = 0; c < nchunks; ++c) s += p[c * E];
    const int r = ent / G, n = ent % G;
    if (r < C) dWx[((int64_t)d * C + r) * G + n] = s;
    else if (r == C) db[(int64_t)d * G + n] = s;
    else if (r < C + 1 + H) dUl[((int64_t)d * H + (r - C - 1)) * G + n] = s;
    else dUu[((int64_t)d * H + (r - C - 1 - H)) * G + n] = s;
}

// one thread per canvas element (pixel, channel): dx inside real pixels, zero elsewhere
__global__ void k_dx(Dev D, int C, int H, const float* __restrict__ Wx, const float* __restrict__ dA,
                     float* __restrict__ dx_flat, float* __restrict__ dx_canvas) {
    const int G = 5 * H;
    const int64_t E = (int64_t)D.Hc * D.Wc * C;
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < E; i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t p = i / C;
        const int ch = (int)(i % C);
        const int e = D.eid[p];
        float v = 0.f;
        bool real = false;
        int64_t fidx = 0;
        if (e >= 0) {
            const int y = (int)(p / D.Wc), x = (int)(p % D.Wc);
            const int ry = y - D.real[4 * e], rx = x - D.real[4 * e + 1];
            const int rw = D.real[4 * e + 3];
            if (ry < D.real[4 * e + 2] && rx < rw) {
                real = true;
                fidx = (D.flat_off[e] + (int64_t)ry * rw + rx) * C + ch;
                const int h = D.rect[4 * e + 2], w = D.rect[4 * e + 3];
                const int ly = y - D.rect[4 * e], lx = x - D.rect[4 * e + 1];
                for (int d = 0; d < 4; ++d) {
                    const int a = (d & 2) ? h - 1 - ly : ly;
                    const int b = (d & 1) ? w - 1 - lx : lx;
                    const int s = a + b;
                    const int64_t cell = (int64_t)d * D.T + D.cell_off[e] + dg_start(h, w, s) + (a - dg_lo(h, w, s));
                    const float* da = dA + cell * G;
                    const float* wr = Wx + ((int64_t)d * C + ch) * G;
                    for (int n = 0; n < G; ++n) v += da[n] * wr[n];
                }
            }
        }
        if (dx_canvas) dx_canvas[i] = v;
        if (dx_flat && real) dx_flat[fidx] = v;
    }
}

}  // namespace

bool wgrad_supported(int C, int H) {
    const int G = 5 * H, R = C + 1 + 2 * H;
    if (G > WG_THREADS) return false;
    const int tpc = WG_THREADS / G;
    return (R + tpc - 1) / tpc <= MAXE;
}

hipError_t launch_wgrad(const Dev& D, const void* x_canvas, int dtype, int C, int H, const float* h_dirs,
                        const float* dA, float* part, int64_t nchunks, float* dWx, float* dUl, float* dUu, float* db,
                        hipStream_t st) {
    const int R = C + 1 + 2 * H, G = 5 * H;
    const size_t lds = sizeof(float) * (size_t)TILE * (R + G);
    const dim3 grid((unsigned)nchunks, 4);
    if (dtype == 0)
        hipLaunchKernelGGL(k_wgrad_partial<float>, grid, dim3(WG_THREADS), lds, st, D, (const float*)x_canvas, C, H,
                           h_dirs, dA, part, nchunks);
    else
        hipLaunchKernelGGL(k_wgrad_partial<uint16_t>, grid, dim3(WG_THREADS), lds, st, D, (const uint16_t*)x_canvas,
                           C, H, h_dirs, dA, part, nchunks);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    const int64_t tot = 4 * (int64_t)R * G;
    hipLaunchKernelGGL(k_wgrad_reduce, dim3((unsigned)((tot + 255) / 256)), dim3(256), 0, st, part, nchunks, C, H, dWx,
                       dUl, dUu, db);
    return hipGetLastError();
}

hipError_t launch_dx(const Dev& D, int C, int H, const float* Wx, const float* dA, float* dx_flat, float* dx_canvas,
                     hipStream_t st) {
    const int64_t E = (int64_t)D.Hc * D.Wc * C;
    int64_t g = (E + 255) / 256;
    if (g > (1 << 20)) g = 1 << 20;
    hipLaunchKernelGGL(k_dx, dim3((unsigned)g), dim3(256), 0, st, D, C, H, Wx, dA, dx_flat, dx_canvas);
    return hipGetLastError();
}

}  // namespace mdl
