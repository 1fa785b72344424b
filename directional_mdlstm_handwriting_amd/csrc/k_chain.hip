// k_chain.hip — the anti-diagonal wavefront recurrence, forward and 2D BPTT.
//
// The dependency structure is that of "No Padding Please" §I/§IV-A and RETURNN
// §4.2: h(u,v) needs h(u-1,v) and h(u,v-1), so all cells of one anti-diagonal
// are independent and are computed together. Because the packer's mask cuts
// every dependency at an example's edge (§V), each example runs on its own
// local diagonals: the number of dependent steps of a pass is max over
// examples of h+w-1 instead of Hc+Wc-1 for the whole canvas.
//
// Work decomposition (gfx950): one workgroup per (example, direction) unit,
// launched in the layout's largest-first order; inside it, one thread per
// (cell of the diagonal, hidden unit k) item, which computes all five gate
// pre-activations of that hidden unit, so a step needs a single barrier.
// The recurrent weights sit in LDS for the whole pass; the previous diagonal's
// (h, c) (forward) or gate gradients (backward) sit in LDS ping-pong buffers.
// Global traffic per step is one contiguous run of the diagonal-major stash
// (prefetched a step ahead in the forward) plus the h output on the canvas.
#include "kernels.h"

namespace mdl {

namespace {

constexpr int CHAIN_THREADS = 256;
constexpr int MAXI = 8;  // (cell, hidden) items per thread and step

__device__ inline float sigm(float z) { return 1.0f / (1.0f + expf(-z)); }

// Forward. Z [4][T][5H], stash out [4][T][6H] = (i, f_l, f_u, o, g, c) per cell,
// h_dirs out [4][Hc][Wc][H].
__global__ __launch_bounds__(CHAIN_THREADS) void k_fwd_chain(Dev D, int H, int Lmax, const float* __restrict__ Ul,
                                                             const float* __restrict__ Uu,
                                                             const float* __restrict__ Z, float* __restrict__ stash,
                                                             float* __restrict__ hdirs) {
    const int u = D.units[blockIdx.x];
    const int e = u >> 2, d = u & 3;
    const Flip F{D.rect[4 * e], D.rect[4 * e + 1], D.rect[4 * e + 2], D.rect[4 * e + 3], (d & 2) != 0, (d & 1) != 0};
    const int h = F.h, w = F.w;
    const int G = 5 * H;
    extern __shared__ float lds[];
    float* U = lds;                  // [2H][G]: rows 0..H-1 = Ul[d], rows H..2H-1 = Uu[d]
    float* hb = U + 2 * H * G;       // [2][Lmax][H]
    float* cb = hb + 2 * Lmax * H;   // [2][Lmax][H]
    for (int i = threadIdx.x; i < H * G; i += blockDim.x) {
        U[i] = Ul[(int64_t)d * H * G + i];
        U[H * G + i] = Uu[(int64_t)d * H * G + i];
    }
    const int64_t base = (int64_t)d * D.T + D.cell_off[e];
    const float* Zd = Z + base * G;
    float* Sd = stash + base * 6 * H;
    float* Hd = hdirs + (int64_t)d * D.Hc * D.Wc * H;
    const int S = h + w - 1;
    const int tid = threadIdx.x, nthr = blockDim.x;

    float zc[MAXI][5];
    {
        const int L = dg_len(h, w, 0);
#pragma unroll
        for (int i = 0; i < MAXI; ++i) {
            const int item = tid + i * nthr;
            if (item < L * H) {
                const int j = item / H, k = item - (item / H) * H;
#pragma unroll
                for (int g = 0; g < 5; ++g) zc[i][g] = Zd[(int64_t)j * G + g * H + k];
            }
        }
    }
    __syncthreads();
    for (int s = 0; s < S; ++s) {
        const int L = dg_len(h, w, s), lo = dg_lo(h, w, s);
        const int64_t st = dg_start(h, w, s);
        const int lop = dg_lo(h, w, s - 1);
        // prefetch the next diagonal's projections
        float zn[MAXI][5];
        if (s + 1 < S) {
            const int Ln = dg_len(h, w, s + 1);
            const int64_t stn = dg_start(h, w, s + 1);
#pragma unroll
            for (int i = 0; i < MAXI; ++i) {
                const int item = tid + i * nthr;
                if (item < Ln * H) {
                    const int j = item / H, k = item - (item / H) * H;
#pragma unroll
                    for (int g = 0; g < 5; ++g) zn[i][g] = Zd[(stn + j) * G + g * H + k];
                }
            }
        }
        const float* hp = hb + ((s + 1) & 1) * Lmax * H;
        const float* cp = cb + ((s + 1) & 1) * Lmax * H;
        float* hn = hb + (s & 1) * Lmax * H;
        float* cn = cb + (s & 1) * Lmax * H;
#pragma unroll
        for (int i = 0; i < MAXI; ++i) {
            const int item = tid + i * nthr;
            if (item < L * H) {
                const int j = item / H, k = item - (item / H) * H;
                const int a = lo + j, b = s - a;
                float acc0 = zc[i][0], acc1 = zc[i][1], acc2 = zc[i][2], acc3 = zc[i][3], acc4 = zc[i][4];
                float cl = 0.f, cu = 0.f;
                if (b > 0) {  // left predecessor (a, b-1) on diagonal s-1
                    const float* hv = hp + (a - lop) * H;
                    const float* Ur = U + k;
                    for (int q = 0; q < H; ++q) {
                        const float x = hv[q];
                        const float* r = Ur + q * G;
                        acc0 += x * r[0];
                        acc1 += x * r[H];
                        acc2 += x * r[2 * H];
                        acc3 += x * r[3 * H];
                        acc4 += x * r[4 * H];
                    }
                    cl = cp[(a - lop) * H + k];
                }
                if (a > 0) {  // upper predecessor (a-1, b) on diagonal s-1
                    const float* hv = hp + (a - 1 - lop) * H;
                    const float* Ur = U + H * G + k;
                    for (int q = 0; q < H; ++q) {
                        const float x = hv[q];
                        const float* r = Ur + q * G;
                        acc0 += x * r[0];
                        acc1 += x * r[H];
                        acc2 += x * r[2 * H];
                        acc3 += x * r[3 * H];
                        acc4 += x * r[4 * H];
                    }
                    cu = cp[(a - 1 - lop) * H + k];
                }
                const float ig = sigm(acc0), fl = sigm(acc1), fu = sigm(acc2), og = sigm(acc3);
                const float gg = tanhf(acc4);
                const float c = fl * cl + fu * cu + ig * gg;
                const float hv = og * tanhf(c);
                hn[j * H + k] = hv;
                cn[j * H + k] = c;
                Hd[((int64_t)F.y(a) * D.Wc + F.x(b)) * H + k] = hv;
                float* rec = Sd + (st + j) * 6 * H + k;
                rec[0] = ig;
                rec[H] = fl;
                rec[2 * H] = fu;
                rec[3 * H] = og;
                rec[4 * H] = gg;
                rec[5 * H] = c;
            }
        }
        __syncthreads();
        if (s + 1 < S) {
#pragma unroll
            for (int i = 0; i < MAXI; ++i)
#pragma unroll
                for (int g = 0; g < 5; ++g) zc[i][g] = zn[i][g];
        }
    }
}

// Backward over the diagonals in reverse. Upstream gradient from dy_flat (same
// for every direction) or dh_dirs [4][Hc][Wc][H]. dA out [4][T][5H].
__global__ __launch_bounds__(CHAIN_THREADS) void k_bwd_chain(Dev D, int H, int Lmax, const float* __restrict__ Ul,
                                                             const float* __restrict__ Uu,
                                                             const float* __restrict__ stash,
                                                             const float* __restrict__ dy_flat,
                                                             const float* __restrict__ dh_dirs,
                                                             float* __restrict__ dA) {
    const int u = D.units[blockIdx.x];
    const int e = u >> 2, d = u & 3;
    const Flip F{D.rect[4 * e], D.rect[4 * e + 1], D.rect[4 * e + 2], D.rect[4 * e + 3], (d & 2) != 0, (d & 1) != 0};
    const int h = F.h, w = F.w;
    const int ry0 = D.real[4 * e], rx0 = D.real[4 * e + 1], rh = D.real[4 * e + 2], rw = D.real[4 * e + 3];
    const int G = 5 * H;
    const int H2 = 2 * H;
    extern __shared__ float lds[];
    float* UT = lds;                  // [G][2H]: UT[n][k] = Ul[d][k][n], UT[n][H+k] = Uu[d][k][n]
    float* dab = UT + G * H2;         // [2][Lmax][G]
    float* dcl = dab + 2 * Lmax * G;  // [2][Lmax][H]  dc * f_l
    float* dcu = dcl + 2 * Lmax * H;  // [2][Lmax][H]  dc * f_u
    for (int i = threadIdx.x; i < H * G; i += blockDim.x) {
        const int k = i / G, n = i - (i / G) * G;
        UT[n * H2 + k] = Ul[(int64_t)d * H * G + i];
        UT[n * H2 + H + k] = Uu[(int64_t)d * H * G + i];
    }
    __syncthreads();
    const int64_t base = (int64_t)d * D.T + D.cell_off[e];
    const float* Sd = stash + base * 6 * H;
    float* dAd = dA + base * G;
    const float* dyb = dy_flat ? dy_flat + D.flat_off[e] * H : nullptr;
    const float* dhd = dh_dirs ? dh_dirs + (int64_t)d * D.Hc * D.Wc * H : nullptr;
    const int S = h + w - 1;
    const int tid = threadIdx.x, nthr = blockDim.x;

    for (int s = S - 1; s >= 0; --s) {
        const int L = dg_len(h, w, s), lo = dg_lo(h, w, s);
        const int64_t st = dg_start(h, w, s);
        const int lon = dg_lo(h, w, s + 1);
        const int lop = s > 0 ? dg_lo(h, w, s - 1) : 0;
        const int64_t stp = s > 0 ? dg_start(h, w, s - 1) : 0;
        const float* dar = dab + ((s + 1) & 1) * Lmax * G;
        const float* dclr = dcl + ((s + 1) & 1) * Lmax * H;
        const float* dcur = dcu + ((s + 1) & 1) * Lmax * H;
        float* daw = dab + (s & 1) * Lmax * G;
        float* dclw = dcl + (s & 1) * Lmax * H;
        float* dcuw = dcu + (s & 1) * Lmax * H;
#pragma unroll
        for (int i = 0; i < MAXI; ++i) {
            const int item = tid + i * nthr;
            if (item < L * H) {
                const int j = item / H, k = item - (item / H) * H;
                const int a = lo + j, b = s - a;
                const int y = F.y(a), x = F.x(b);
                // forward values of this cell and its predecessors' memory states
                const float* rec = Sd + (st + j) * 6 * H + k;
                const float ig = rec[0], fl = rec[H], fu = rec[2 * H], og = rec[3 * H], gg = rec[4 * H];
                const float c = rec[5 * H];
                const float cl = b > 0 ? Sd[(stp + a - lop) * 6 * H + 5 * H + k] : 0.f;
                const float cu = a > 0 ? Sd[(stp + a - 1 - lop) * 6 * H + 5 * H + k] : 0.f;
                float dh = 0.f;
                if (dhd) {
                    dh = dhd[((int64_t)y * D.Wc + x) * H + k];
                } else {
                    const int ly = y - ry0, lx = x - rx0;
                    if (ly < rh && lx < rw) dh = dyb[((int64_t)ly * rw + lx) * H + k];
                }
                float dcin = 0.f;
                if (b + 1 < w) {  // right successor (a, b+1): this cell is its left predecessor
                    const int jr = a - lon;
                    const float* dv = dar + jr * G;
                    const float* ut = UT + k;
                    for (int n = 0; n < G; ++n) dh += dv[n] * ut[n * H2];
                    dcin += dclr[jr * H + k];
                }
                if (a + 1 < h) {  // lower successor (a+1, b): this cell is its upper predecessor
                    const int jd = a + 1 - lon;
                    const float* dv = dar + jd * G;
                    const float* ut = UT + H + k;
                    for (int n = 0; n < G; ++n) dh += dv[n] * ut[n * H2];
                    dcin += dcur[jd * H + k];
                }
                const float tc = tanhf(c);
                const float dov = dh * tc;
                const float dc = dcin + dh * og * (1.f - tc * tc);
                const float d0 = dc * gg * ig * (1.f - ig);
                const float d1 = dc * cl * fl * (1.f - fl);
                const float d2 = dc * cu * fu * (1.f - fu);
                const float d3 = dov * og * (1.f - og);
                const float d4 = dc * ig * (1.f - gg * gg);
                float* dw = daw + j * G + k;
                dw[0] = d0; dw[H] = d1; dw[2 * H] = d2; dw[3 * H] = d3; dw[4 * H] = d4;
                dclw[j * H + k] = dc * fl;
                dcuw[j * H + k] = dc * fu;
                float* dg = dAd + (st + j) * G + k;
                dg[0] = d0; dg[H] = d1; dg[2 * H] = d2; dg[3 * H] = d3; dg[4 * H] = d4;
            }
        }
        __syncthreads();
    }
}

}  // namespace

int chain_max_items() { return MAXI * CHAIN_THREADS; }

size_t fwd_chain_lds(int H, int Lmax) {
    return sizeof(float) * ((size_t)2 * H * 5 * H + (size_t)4 * Lmax * H);
}

size_t bwd_chain_lds(int H, int Lmax) {
    return sizeof(float) * ((size_t)2 * H * 5 * H + (size_t)2 * Lmax * 5 * H + (size_t)4 * Lmax * H);
}

hipError_t launch_fwd_chain(const Dev& D, int H, const float* Ul, const float* Uu, const float* Z, float* stash,
                            float* h_dirs, hipStream_t st) {
    const int Lmax = D.max_diag;
    hipLaunchKernelGGL(k_fwd_chain, dim3(4 * D.n), dim3(CHAIN_THREADS), fwd_chain_lds(H, Lmax), st, D, H, Lmax, Ul,
                       Uu, Z, stash, h_dirs);
    return hipGetLastError();
}

hipError_t launch_bwd_chain(const Dev& D, int H, const float* Ul, const float* Uu, const float* stash,
                            const float* dy_flat, const float* dh_dirs, float* dA, hipStream_t st) {
    const int Lmax = D.max_diag;
    hipLaunchKernelGGL(k_bwd_chain, dim3(4 * D.n), dim3(CHAIN_THREADS), bwd_chain_lds(H, Lmax), st, D, H, Lmax, Ul,
                       Uu, stash, dy_flat, dh_dirs, dA);
    return hipGetLastError();
}

}  // namespace mdl
