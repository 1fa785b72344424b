// k_conv.hip — block-strided convolution between MDLSTM levels on packed canvases.
//
// "No Padding Please", §V-B: the kernel's stride equals its size, so every
// output pixel reads its own kh x kw block; tensor-list chunking stacks all
// blocks of all examples and runs one convolution over them, and de-chunking
// puts each example's outputs back by its size. Here the chunks never leave
// the canvases: output pixels of the level-(k+1) canvas are taken in tiles of
// CW_TILE, each tile's blocks (all four directions' hidden outputs of the
// level-k canvas, 4H channels) are gathered into LDS once, and the products
// run from there:
//   forward   x1[p][o] = bc[o] + sum_f Wc[o][f] blk[p][f]     (Wc staged in LDS as well)
//   dW, db    partial sums over the tiles of a chunk of output pixels, per
//             workgroup, then added in chunk order (fixed order, no atomics)
// with f = ((d H + k) kh + i) kw + j, the layout of Wc's trailing axes, and
// block elements outside the level-k example read as zero (partial blocks at
// the bottom and right edge are zero-padded). The data gradient scatters the
// output gradient back through the same blocks, one thread per element of dh
// (Wc staged in LDS).
#include "kernels.h"

#include <mutex>

namespace mdl {

namespace {

constexpr int CW_THREADS = 512;
constexpr int CW_MAXE = 16;   // weight-gradient entries per thread: Cout (K + 1) <= CW_MAXE CW_THREADS
constexpr int CW_TILE = 16;   // output pixels per staged tile
constexpr int CW_GROUPS = 512;  // at most this many weight-gradient workgroups (chunks)

// Where output pixel p1 of the level-(k+1) canvas takes its block: the block's first level-k pixel
// (row-major index on the level-k canvas), the rows and columns of the block inside the level-k example
// (0 rows for a pixel outside every example's real region, whose block is all zero).
struct BlockSrc {
    int base, nrow, ncol;
};

__device__ inline BlockSrc block_src(const Dev& Dk, const Dev& Dk1, int64_t p1, int kh, int kw) {
    BlockSrc b{0, 0, 0};
    const int e = Dk1.eid[p1];
    if (e < 0) return b;
    const int r = (int)(p1 / Dk1.Wc) - Dk1.real[4 * e];
    const int c = (int)(p1 % Dk1.Wc) - Dk1.real[4 * e + 1];
    if (r >= Dk1.real[4 * e + 2] || c >= Dk1.real[4 * e + 3]) return b;
    const int yy = kh * r, xx = kw * c;
    b.base = (Dk.real[4 * e] + yy) * Dk.Wc + Dk.real[4 * e + 1] + xx;
    b.nrow = min(kh, Dk.real[4 * e + 2] - yy);
    b.ncol = min(kw, Dk.real[4 * e + 3] - xx);
    return b;
}

// Gathers the blocks of output pixels [p0, p0 + CW_TILE) into blk[CW_TILE][KS] (row stride KS >= K; zero
// past P1), using the per-pixel sources `src` the caller filled. Consecutive threads take consecutive f.
__device__ inline void gather_tile(const Dev& Dk, const float* __restrict__ hk, int H, int kh, int kw, int K, int KS,
                                   const BlockSrc* src, float* blk) {
    const int64_t plane = (int64_t)Dk.Hc * Dk.Wc * H;
    for (int idx = threadIdx.x; idx < CW_TILE * K; idx += blockDim.x) {
        const int tt = idx / K, f = idx - tt * K;
        const int j = f % kw, i = (f / kw) % kh, k = (f / (kw * kh)) % H, d = f / (kw * kh * H);
        const BlockSrc s = src[tt];
        float v = 0.f;
        if (i < s.nrow && j < s.ncol) v = hk[d * plane + (int64_t)(s.base + i * Dk.Wc + j) * H + k];
        blk[tt * KS + f] = v;
    }
}

// Forward: workgroups stride over tiles of CW_TILE canvas pixels of level k+1; Wc [Cout][K] sits in LDS
// for the whole workgroup. Every canvas pixel is written (zero outside the real pixels).
__global__ __launch_bounds__(256) void k_conv_fwd(Dev Dk, Dev Dk1, const float* __restrict__ hk, int H, int kh,
                                                  int kw, const float* __restrict__ Wc,
                                                  const float* __restrict__ bc, int Cout, float* __restrict__ x1) {
    const int K = 4 * H * kh * kw;
    const int KS = K | 1;  // odd row stride: the lanes of a wave read different rows on different banks
    extern __shared__ float lds[];
    float* w = lds;                         // [Cout][KS]
    float* blk = w + Cout * KS;             // [CW_TILE][KS]
    BlockSrc* src = reinterpret_cast<BlockSrc*>(blk + CW_TILE * KS);  // [CW_TILE]
    for (int i = threadIdx.x; i < Cout * K; i += blockDim.x) w[(i / K) * KS + i % K] = Wc[i];
    const int64_t P1 = (int64_t)Dk1.Hc * Dk1.Wc;
    const int64_t ntiles = (P1 + CW_TILE - 1) / CW_TILE;
    for (int64_t tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
        const int64_t p0 = tile * CW_TILE;
        __syncthreads();  // the previous tile's reads of blk and src are done
        if (threadIdx.x < CW_TILE) {
            const int64_t p1 = p0 + threadIdx.x;
            src[threadIdx.x] = p1 < P1 ? block_src(Dk, Dk1, p1, kh, kw) : BlockSrc{0, 0, 0};
        }
        __syncthreads();
        gather_tile(Dk, hk, H, kh, kw, K, KS, src, blk);
        __syncthreads();
        for (int o2 = threadIdx.x; o2 < CW_TILE * Cout; o2 += blockDim.x) {
            const int tt = o2 / Cout, o = o2 - tt * Cout;
            const int64_t p1 = p0 + tt;
            if (p1 >= P1) continue;
            float v = 0.f;
            if (src[tt].nrow > 0) {
                v = bc[o];
                const float* br = blk + tt * KS;
                const float* wr = w + o * KS;
                for (int f = 0; f < K; ++f) v += wr[f] * br[f];
            }
            x1[p1 * Cout + o] = v;
        }
    }
}

// Data gradient: one thread per element of dh_k [4][Hc][Wc][H], workgroups striding over them; Wc sits in
// LDS transposed to [f][Cout] (row stride Cout | 1), so a thread's Cout weights are consecutive.
__global__ __launch_bounds__(256) void k_conv_bwd_data(Dev Dk, Dev Dk1, int H, int kh, int kw,
                                                       const float* __restrict__ Wc, int Cout,
                                                       const float* __restrict__ dx1, float* __restrict__ dhk) {
    const int K = 4 * H * kh * kw;
    const int CS = Cout | 1;
    extern __shared__ float wt[];  // [K][CS]
    for (int i = threadIdx.x; i < Cout * K; i += blockDim.x) wt[(i % K) * CS + i / K] = Wc[i];
    __syncthreads();
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
                const float* wr = wt + (((d * H + k) * kh + i) * kw + j) * CS;
                for (int o = 0; o < Cout; ++o) v += g[o] * wr[o];
            }
        }
        dhk[t] = v;
    }
}

// Output pixels per weight-gradient chunk: whole tiles, at most CW_GROUPS chunks over the level-(k+1)
// canvas.
inline int64_t conv_chunk(const Dev& Dk1) {
    const int64_t P1 = (int64_t)Dk1.Hc * Dk1.Wc;
    const int64_t per = (P1 + CW_GROUPS - 1) / CW_GROUPS;
    return (per + CW_TILE - 1) / CW_TILE * CW_TILE;
}

// grid nchunks: partial sums of dWc (and dbc) over one chunk of level-(k+1) canvas pixels (pixels outside
// the real pixels carry a zero gradient and an all-zero block)
__global__ __launch_bounds__(CW_THREADS) void k_conv_wpartial(Dev Dk, Dev Dk1, const float* __restrict__ hk, int H,
                                                              int kh, int kw, int Cout, const float* __restrict__ dx1,
                                                              int64_t chunk, float* __restrict__ part) {
    const int K = 4 * H * kh * kw;
    const int E = Cout * (K + 1);
    const int64_t P1 = (int64_t)Dk1.Hc * Dk1.Wc;
    const int64_t q0 = (int64_t)blockIdx.x * chunk;
    const int64_t q1 = q0 + chunk < P1 ? q0 + chunk : P1;
    extern __shared__ float lds[];
    float* blk = lds;                   // [CW_TILE][K]
    float* gx = blk + CW_TILE * K;      // [CW_TILE][Cout]
    BlockSrc* src = reinterpret_cast<BlockSrc*>(gx + CW_TILE * Cout);  // [CW_TILE]
    const int tid = threadIdx.x, nthr = blockDim.x;
    float acc[CW_MAXE];
#pragma unroll
    for (int i = 0; i < CW_MAXE; ++i) acc[i] = 0.f;
    for (int64_t t0 = q0; t0 < q1; t0 += CW_TILE) {
        if (tid < CW_TILE) {
            const int64_t p1 = t0 + tid;
            src[tid] = p1 < q1 ? block_src(Dk, Dk1, p1, kh, kw) : BlockSrc{0, 0, 0};
        }
        __syncthreads();
        gather_tile(Dk, hk, H, kh, kw, K, K, src, blk);
        for (int idx = tid; idx < CW_TILE * Cout; idx += nthr) {
            const int tt = idx / Cout;
            gx[idx] = src[tt].nrow > 0 ? dx1[(t0 + tt) * Cout + (idx - tt * Cout)] : 0.f;
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

// dWc and dbc: the chunk partials summed in a fixed order. A workgroup takes 64 consecutive entries and 16
// slices of the chunks (slice j adds chunks j, j + 16, ... in order); the slice sums are then added in
// slice order.
constexpr int CR_X = 64, CR_Y = 16;
__global__ __launch_bounds__(CR_X* CR_Y) void k_conv_wreduce(const float* __restrict__ part, int64_t nchunks, int K,
                                                             int Cout, float* __restrict__ dWc,
                                                             float* __restrict__ dbc) {
    const int E = Cout * (K + 1);
    const int tx = threadIdx.x % CR_X, ty = threadIdx.x / CR_X;
    const int id = blockIdx.x * CR_X + tx;
    float s = 0.f;
    if (id < E)
        for (int64_t c = ty; c < nchunks; c += CR_Y) s += part[c * E + id];
    __shared__ float red[CR_Y][CR_X];
    red[ty][tx] = s;
    __syncthreads();
    if (ty != 0 || id >= E) return;
    float t = red[0][tx];
#pragma unroll
    for (int y = 1; y < CR_Y; ++y) t += red[y][tx];
    const int o = id / (K + 1), f = id % (K + 1);
    if (f < K) dWc[(int64_t)o * K + f] = t; else dbc[o] = t;
}

inline unsigned grid_for(int64_t n) {
    int64_t g = (n + 255) / 256;
    if (g < 1) g = 1;
    return (unsigned)(g < (1 << 20) ? g : (1 << 20));
}

}  // namespace

// The weight-gradient partials of the entry point that allocates nothing: one fixed array per device, as large
// as the partials of any accepted call (at most CW_GROUPS chunks of Cout (K + 1) <= CW_MAXE CW_THREADS floats),
// resident for the life of the process. Its device address is looked up once per device, with that device
// current; host code passes that address, never the symbol itself.
constexpr size_t kConvScratchFloats = (size_t)CW_GROUPS * CW_MAXE * CW_THREADS;  // 16 MiB
static __device__ __align__(256) float scratch[kConvScratchFloats];

hipError_t conv_scratch(void** ptr, size_t* bytes) {
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static void* addr[kMaxDevices] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lk(mu);
    if (!addr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        addr[dev] = p;
    }
    *ptr = addr[dev];
    *bytes = kConvScratchFloats * sizeof(float);
    return hipSuccess;
}

int64_t conv_nchunks(const Dev& Dk1) {
    const int64_t P1 = (int64_t)Dk1.Hc * Dk1.Wc;
    const int64_t c = conv_chunk(Dk1);
    return (P1 + c - 1) / c;
}

size_t conv_fwd_lds(int H, int kh, int kw, int Cout) {
    const size_t KS = (4 * (size_t)H * kh * kw) | 1;
    return sizeof(float) * ((size_t)Cout * KS + CW_TILE * KS) + sizeof(BlockSrc) * CW_TILE;
}

size_t conv_data_lds(int H, int kh, int kw, int Cout) {
    return sizeof(float) * 4 * (size_t)H * kh * kw * (size_t)(Cout | 1);
}

size_t conv_wgrad_lds(int H, int kh, int kw, int Cout) {
    const size_t K = 4 * (size_t)H * kh * kw;
    return sizeof(float) * (CW_TILE * K + CW_TILE * (size_t)Cout) + sizeof(BlockSrc) * CW_TILE;
}

hipError_t launch_conv_fwd(const Dev& Dk, const Dev& Dk1, const float* h_dirs_k, int H, int kh, int kw,
                           const float* Wc, const float* bc, int Cout, float* x_k1, hipStream_t st) {
    const int64_t ntiles = ((int64_t)Dk1.Hc * Dk1.Wc + CW_TILE - 1) / CW_TILE;
    const unsigned grid = (unsigned)(ntiles < 1024 ? ntiles : 1024);
    launch(k_conv_fwd, dim3(grid), dim3(256), conv_fwd_lds(H, kh, kw, Cout), st, Dk, Dk1, h_dirs_k, H, kh, kw, Wc,
           bc, Cout, x_k1);
    return hipGetLastError();
}

hipError_t launch_conv_bwd(const Dev& Dk, const Dev& Dk1, const float* h_dirs_k, int H, int kh, int kw,
                           const float* Wc, int Cout, const float* dx_k1, float* dh_k, float* dWc, float* dbc,
                           float* part, hipStream_t st) {
    const int64_t E = 4 * (int64_t)Dk.Hc * Dk.Wc * H;
    const unsigned gd = grid_for(E) < 2048 ? grid_for(E) : 2048;  // each workgroup stages Wc once
    launch(k_conv_bwd_data, dim3(gd), dim3(256), conv_data_lds(H, kh, kw, Cout), st, Dk, Dk1, H, kh, kw, Wc, Cout,
           dx_k1, dh_k);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    const int K = 4 * H * kh * kw;
    const int64_t nch = conv_nchunks(Dk1);
    launch(k_conv_wpartial, dim3((unsigned)nch), dim3(CW_THREADS), conv_wgrad_lds(H, kh, kw, Cout), st, Dk, Dk1,
           h_dirs_k, H, kh, kw, Cout, dx_k1, conv_chunk(Dk1), part);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
    const int Ew = Cout * (K + 1);
    launch(k_conv_wreduce, dim3((Ew + CR_X - 1) / CR_X), dim3(CR_X * CR_Y), 0, st, part, nch, K, Cout, dWc, dbc);
    return hipGetLastError();
}

}  // namespace mdl
