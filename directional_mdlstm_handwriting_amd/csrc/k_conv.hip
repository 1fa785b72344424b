// k_conv.hip — block-strided convolution between MDLSTM levels on packed canvases.
//
// "No Padding Please", §V-B: the kernel's stride equals its size, so every
// output pixel reads its own kh x kw block; tensor-list chunking stacks all
// blocks of all examples and runs one convolution over them, and de-chunking
// puts each example's outputs back by its size. Here the chunks never leave
// the canvases: each output pixel of the level-(k+1) canvas gathers its block
// from the level-k canvas (all four directions' hidden outputs as 4H
// channels), one output channel per thread; the backward scatters the output
// gradient back through the same blocks. Weight gradients are fixed-order
// chunked sums over the output pixels. These kernels move little data and are
// HBM/latency bound.
#include "kernels.h"

namespace mdl {

namespace {

constexpr int CONV_CHUNK = 1024;  // output pixels per weight-gradient partial sum
constexpr int CW_THREADS = 512;
constexpr int CW_MAXE = 16;
constexpr int CW_TILE = 16;

// one thread per (level-(k+1) canvas pixel, output channel)
__global__ void k_conv_fwd(Dev Dk, Dev Dk1, const float* __restrict__ hk, int H, int kh, int kw,
                           const float* __restrict__ Wc, const float* __restrict__ bc, int Cout,
                           float* __restrict__ x1) {
    const int64_t E = (int64_t)Dk1.Hc * Dk1.Wc * Cout;
    const int64_t plane = (int64_t)Dk.Hc * Dk.Wc * H;
    for (int64_t t = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; t < E; t += (int64_t)gridDim.x * blockDim.x) {
        const int64_t p1 = t / Cout;
        const int o = (int)(t % Cout);
        const int e = Dk1.eid[p1];
        float v = 0.f;
        if (e >= 0) {
            const int r = (int)(p1 / Dk1.Wc) - Dk1.real[4 * e];
            const int c = (int)(p1 % Dk1.Wc) - Dk1.real[4 * e + 1];
            if (r < Dk1.real[4 * e + 2] && c < Dk1.real[4 * e + 3]) {
                const int y0 = Dk.real[4 * e], x0 = Dk.real[4 * e + 1], h = Dk.real[4 * e + 2], w = Dk.real[4 * e + 3];
                v = bc[o];
                for (int d = 0; d < 4; ++d)
                    for (int k = 0; k < H; ++k) {
                        const float* wr = Wc + (((int64_t)o * 4 + d) * H + k) * kh * kw;
                        for (int i = 0; i < kh; ++i) {
                            const int yy = kh * r + i;
                            if (yy >= h) break;
                            for (int j = 0; j < kw; ++j) {
                                const int xx = kw * c + j;
                                if (xx >= w) break;
                                v += wr[i * kw + j] * hk[d * plane + ((int64_t)(y0 + yy) * Dk.Wc + x0 + xx) * H + k];
                            }
                        }
                    }
            }
        }
        x1[t] = v;
    }
}

// one thread per element of dh_k [4][Hc][Wc][H]
__global__ void k_conv_bwd_data(Dev Dk, Dev Dk1, int H, int kh, int kw, const float* __restrict__ Wc, int Cout,
                                const float* __restrict__ dx1, float* __restrict__ dhk) {
    const int64_t P = (int64_t)Dk.Hc * Dk.Wc;
    const int64_t E = 4 * P * H;
    for (int64_t t = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; t < E; t += (int64_t)gridDim.x * blockDim.x) {
        const int d = (int)(t / (P * H));
        const int64_t rem = t - (int64_t)d * P * H;
        const int64_t p = rem / H;
        const int k = (int)(rem % H);
        const int e = Dk.eid[p];
        float v = 0.f;
        if (e >= 0) {
            const int ly = (int)(p / Dk.Wc) - Dk.real[4 * e];
            const int lx = (int)(p % Dk.Wc) - Dk.real[4 * e + 1];
            if (ly < Dk.real[4 * e + 2] && lx < Dk.real[4 * e + 3]) {
                const int r = ly / kh, i = ly - r * kh, c = lx / kw, j = lx - c * kw;
                const int64_t p1 = (int64_t)(Dk1.real[4 * e] + r) * Dk1.Wc + Dk1.real[4 * e + 1] + c;
                const float* g = dx1 + p1 * Cout;
                for (int o = 0; o < Cout; ++o)
                    v += g[o] * Wc[((((int64_t)o * 4 + d) * H + k) * kh + i) * kw + j];
            }
        }
        dhk[t] = v;
    }
}

// grid nchunks: partial sums of dWc (and dbc) over CONV_CHUNK consecutive real output pixels
__global__ __launch_bounds__(CW_THREADS) void k_conv_wpartial(Dev Dk, Dev Dk1, const float* __restrict__ hk, int H,
                                                              int kh, int kw, int Cout, const float* __restrict__ dx1,
                                                              float* __restrict__ part) {
    const int K = 4 * H * kh * kw;
    const int E = Cout * (K + 1);
    const int64_t q0 = (int64_t)blockIdx.x * CONV_CHUNK;
    const int64_t q1 = q0 + CONV_CHUNK < Dk1.N ? q0 + CONV_CHUNK : Dk1.N;
    const int64_t plane = (int64_t)Dk.Hc * Dk.Wc * H;
    extern __shared__ float lds[];
    float* blk = lds;                   // [CW_TILE][K]
    float* gx = blk + CW_TILE * K;      // [CW_TILE][Cout]
    const int tid = threadIdx.x, nthr = blockDim.x;
    float acc[CW_MAXE];
#pragma unroll
    for (int i = 0; i < CW_MAXE; ++i) acc[i] = 0.f;
    for (int64_t t0 = q0; t0 < q1; t0 += CW_TILE) {
        for (int idx = tid; idx < CW_TILE * (K + Cout); idx += nthr) {
            const int tt = idx / (K + Cout), f = idx - tt * (K + Cout);
            const int64_t q = t0 + tt;
            float v = 0.f;
            if (q < q1) {
                const int e = find_example(Dk1.flat_off, Dk1.n, q);
                const int w1 = Dk1.real[4 * e + 3];
                const int64_t qq = q - Dk1.flat_off[e];
                const int r = (int)(qq / w1), c = (int)(qq % w1);
                if (f < K) {
                    const int j = f % kw, i = (f / kw) % kh, k = (f / (kw * kh)) % H, d = f / (kw * kh * H);
                    const int yy = kh * r + i, xx = kw * c + j;
                    if (yy < Dk.real[4 * e + 2] && xx < Dk.real[4 * e + 3])
                        v = hk[d * plane + ((int64_t)(Dk.real[4 * e] + yy) * Dk.Wc + Dk.real[4 * e + 1] + xx) * H + k];
                } else {
                    const int64_t p1 = (int64_t)(Dk1.real[4 * e] + r) * Dk1.Wc + Dk1.real[4 * e + 1] + c;
                    v = dx1[p1 * Cout + (f - K)];
                }
            }
            if (f < K) blk[tt * K + f] = v; else gx[tt * Cout + (f - K)] = v;
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < CW_MAXE; ++i) {
            const int ent = tid + i * nthr;
            if (ent < E) {
                const int o = ent / (K + 1), f = ent - o * (K + 1);
                float s = acc[i];
                if (f < K)
                    for (int tt = 0; tt < CW_TILE; ++tt) s += gx[tt * Cout + o] * blk[tt * K + f];
                else
                    for (int tt = 0; tt < CW_TILE; ++tt) s += gx[tt * Cout + o];
                acc[i] = s;
            }
        }
        __syncthreads();
    }
    float* out = part + (int64_t)blockIdx.x * E;
#pragma unroll
    for (int i = 0; i < CW_MAXE; ++i) {
        const int ent = tid + i * nthr;
        if (ent < E) out[ent] = acc[i];
    }
}

__global__ void k_conv_wreduce(const float* __restrict__ part, int64_t nchunks, int K, int Cout,
                               float* __restrict__ dWc, float* __restrict__ dbc) {
    const int E = Cout * (K + 1);
    const int id = blockIdx.x * blockDim.x + threadIdx.x;
    if (id >= E) return;
    float s = 0.f;
    for (int64_t c = 0; c < nchunks; ++c) s += part[c * E + id];
    const int o = id / (K + 1), f = id % (K + 1);
    if (f < K) dWc[(int64_t)o * K + f] = s; else dbc[o] = s;
}

inline unsigned grid_for(int64_t n) {
    int64_t g = (n + 255) / 256;
    if (g < 1) g = 1;
    return (unsigned)(g < (1 << 20) ? g : (1 << 20));
}

}  // namespace

int64_t conv_nchunks(const Dev& Dk1) { return (Dk1.N + CONV_CHUNK - 1) / CONV_CHUNK; }

hipError_t launch_conv_fwd(const Dev& Dk, const Dev& Dk1, const float* h_dirs_k, int H, int kh, int kw,
                           const float* Wc, const float* bc, int Cout, float* x_k1, hipStream_t st) {
    const int64_t E = (int64_t)Dk1.Hc * Dk1.Wc * Cout;
    launch(k_conv_fwd, dim3(grid_for(E)), dim3(256), 0, st, Dk, Dk1, h_dirs_k, H, kh, kw, Wc, bc, Cout,
           x_k1);
    return hipGetLastError();
}

hipError_t launch_conv_bwd(const Dev& Dk, const Dev& Dk1, const float* h_dirs_k, int H, int kh, int kw,
                           const float* Wc, int Cout, const float* dx_k1, float* dh_k, float* dWc, float* dbc,
                           float* part, hipStream_t st) {
    const int64_t E = 4 * (int64_t)Dk.Hc * Dk.Wc * H;
    launch(k_conv_bwd_data, dim3(grid_for(E)), dim3(256), 0, st, Dk, Dk1, H, kh, kw, Wc, Cout, dx_k1,
           dh_k);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    const int K = 4 * H * kh * kw;
    const int64_t nch = conv_nchunks(Dk1);
    const size_t lds = sizeof(float) * (size_t)CW_TILE * (K + Cout);
    launch(k_conv_wpartial, dim3((unsigned)nch), dim3(CW_THREADS), lds, st, Dk, Dk1, h_dirs_k, H, kh, kw,
           Cout, dx_k1, part);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
    const int Ew = Cout * (K + 1);
    launch(k_conv_wreduce, dim3((Ew + 255) / 256), dim3(256), 0, st, part, nch, K, Cout, dWc, dbc);
    return hipGetLastError();
}

}  // namespace mdl
