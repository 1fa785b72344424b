// k_wgrad.hip — weight and input gradients after the reverse wavefront.
//
// RETURNN §4.2: after the recurrent part is back-propagated through time, the
// gradients with respect to the weights and the inputs are matrix products
// over the whole batch. For direction d, with the A-row of a computed cell p
//     r(p) = [x(p), 1, h_left(p), h_up(p)]      (C + 1 + 2H values; a predecessor
//                                              outside the example reads as zero)
// and its gate gradient da_d(p) (5H values):
//     [dWx; db; dUl; dUu][d] = sum over computed cells p of r(p)^T da_d(p)
//     dx(p)                  = sum over d of da_d(p) Wx[d]^T
// One workgroup takes one segment of the layout's weight-gradient split (a
// range of cells of one example) for all four directions: it stages tiles of
// TP cells of A-rows and gate gradients in LDS, accumulates r^T da on the
// matrix cores (v_mfma_f32_16x16x4_f32, K = cells, fp32 products and sums;
// wave d owns direction d's output tiles, up to 32 per pass over the segment),
// and computes dx of the same cells from the staged gate gradients. Segment
// partial sums are then added in segment order by a second kernel, so the
// result is bit-reproducible.
#include "kernels.h"
#include "devmath.h"

namespace mdl {

WsLayout ws_layout(int64_t T, int64_t nparts, int C, int H) {
    auto al = [](size_t v) { return (v + 255) & ~size_t(255); };
    WsLayout w;
    const int G = 5 * H;
    const int R = C + 1 + 2 * H;
    w.nparts = nparts;
    size_t p = 0;
    w.stash = p; p = al(p + sizeof(float) * 4 * (size_t)T * 6 * H);
    w.zda = p;   p = al(p + sizeof(float) * 4 * (size_t)T * G);
    w.part = p;  p = al(p + sizeof(float) * 4 * (size_t)nparts * R * G);
    w.total = p;
    return w;
}

namespace {

constexpr int ACC_TILES = 16;   // 16x16 output tiles one wave owns per pass
constexpr int STAGE_H = 4096;   // staged predecessor-h values per tile (all directions)
constexpr int STAGE_D = 10240;  // staged gate-gradient values per tile (all directions)

constexpr int kOOB = 0x7ffffff0;  // byte offset past every buffer range: loads return 0

// n / d for n < 2^16, d < 2^16, with m = 2^32 / d + 1
__host__ __device__ inline uint32_t magic(uint32_t d) { return (uint32_t)(0xffffffffu / d) + 1u; }
__device__ inline int fdiv(int n, uint32_t m) { return (int)__umulhi((uint32_t)n, m); }

struct WgradShape {
    int C, H, G, R, MT, NT, Q, P, TP;  // Q N-tiles per pass, P passes over the segment, TP cells per tile
    int nh, nd, nx;                  // staged elements per tile: predecessor h, gate gradients, x
    uint32_t m_hd, m_h2, m_gd, m_g, m_x;
    int wx_lds;                      // Wx copied to LDS
    int sp;                          // threads per dx output
};

__host__ __device__ inline size_t wgrad_lds_floats(const WgradShape& s) {
    return (size_t)s.nx + s.nh + s.nd + 4 * (size_t)s.TP * s.C + 1;
}

inline WgradShape wgrad_shape(int C, int H) {
    WgradShape s;
    s.C = C;
    s.H = H;
    s.G = 5 * H;
    s.R = C + 1 + 2 * H;
    s.MT = (s.R + 15) / 16;
    s.NT = (s.G + 15) / 16;
    s.Q = ACC_TILES / s.MT < 1 ? 1 : ACC_TILES / s.MT;   // N-tiles per pass (all M-tiles each pass)
    if (s.Q > s.NT) s.Q = s.NT;
    s.P = (s.NT + s.Q - 1) / s.Q;
    s.TP = 32;
    while (s.TP > 4 && (4 * s.TP * 2 * H > STAGE_H || 4 * s.TP * s.G > STAGE_D)) s.TP /= 2;
    s.nh = 4 * s.TP * 2 * H;
    s.nd = 4 * s.TP * s.G;
    s.nx = s.TP * (C + 1);
    s.m_hd = magic(s.TP * 2 * H);
    s.m_h2 = magic(2 * H);
    s.m_gd = magic(s.TP * s.G);
    s.m_g = magic(s.G);
    s.m_x = magic(C + 1);
    s.wx_lds = 0;
    s.sp = 1;
    return s;
}

// position of region-local cell (ly, lx) of an h x w region in direction d's diagonal-major order
__device__ inline int stash_index(int h, int w, int ly, int lx, int d) {
    const int a = (d & 2) ? h - 1 - ly : ly;
    const int b = (d & 1) ? w - 1 - lx : lx;
    const int s = a + b;
    return (int)dg_start(h, w, s) + (a - dg_lo(h, w, s));
}

// CT/HT > 0: channel count and hidden size fixed at compile time (loops unroll, divisions fold);
// 0: taken from the shape at run time.
template <bool BF16, int CT, int HT>
__global__ __launch_bounds__(256) void k_wgrad_mfma(Dev D, const void* __restrict__ xc, WgradShape S,
                                                    const float* __restrict__ hdirs, const float* __restrict__ dA,
                                                    const float* __restrict__ Wx, float* __restrict__ part,
                                                    float* __restrict__ dx_flat, float* __restrict__ dx_canvas) {
    constexpr int MAXH = STAGE_H / 256, MAXD = STAGE_D / 256, MAXX = 2;
    const int C = CT > 0 ? CT : S.C, H = HT > 0 ? HT : S.H;
    const int G = 5 * H, R = C + 1 + 2 * H, H2 = 2 * H;
    const int MT = (R + 15) / 16, NT = (G + 15) / 16;
    const int TP = S.TP;
    const int ch = blockIdx.x;
    const int e = D.segs[3 * ch], c0 = D.segs[3 * ch + 1], c1 = D.segs[3 * ch + 2];
    const int y0 = D.rect[4 * e], x0 = D.rect[4 * e + 1], h = D.rect[4 * e + 2], w = D.rect[4 * e + 3];
    const int ry0 = D.real[4 * e], rx0 = D.real[4 * e + 1], rh = D.real[4 * e + 2], rw = D.real[4 * e + 3];
    const int tid = threadIdx.x;
    const int lane = tid & 63, wd = tid >> 6;      // wave wd: direction wd
    const int l16 = lane & 15, krow = lane >> 4;
    extern __shared__ float lds[];
    float* xs = lds;                               // [TP][C+1]  x and the constant 1
    float* hs = xs + S.nx;                         // [4][TP][2H] h_left, h_up
    float* dab = hs + S.nh;                        // [4][TP][G]  gate gradients
    float* dxs = dab + S.nd;                       // [4][TP][C]  per-direction dx
    float* zero = dxs + 4 * TP * C;                // one 0.0f
    __shared__ int t_pix[32], t_flat[32], t_cst[4][32], t_flags[32];
    if (tid == 0) zero[0] = 0.f;
    // dx B fragments: Wx[d][c][n] as B[n = 4ks + krow][c = l16]; kept in registers for the whole segment
    // when the shape is fixed at compile time with C <= 16, else loaded per use
    constexpr bool PRE = CT > 0 && CT <= 16 && HT > 0;
    constexpr int KX = HT > 0 ? (5 * HT + 3) / 4 : 64;
    float bwx[PRE ? KX : 1];
    if (PRE) {
#pragma unroll
        for (int ks = 0; ks < (PRE ? KX : 1); ++ks) {
            const int n = 4 * ks + krow;
            bwx[ks] = (l16 < C && n < G) ? Wx[((int64_t)wd * C + l16) * G + n] : 0.f;
        }
    }
    const int plane = D.Hc * D.Wc * H;
    const float* xf = static_cast<const float*>(xc);
    const uint16_t* xb = static_cast<const uint16_t*>(xc);
    const __amdgpu_buffer_rsrc_t rH = rsrc(hdirs, 4 * (int64_t)plane * 4);
    const __amdgpu_buffer_rsrc_t rA = rsrc(dA, 4 * D.T * G * 4);
    const int ncell = c1 - c0;
    const int cell0 = (int)D.cell_off[e];

    // passes over the segment: all MT M-tiles times NQ N-tiles at a time
    constexpr int MTC = HT > 0 ? (CT + 1 + 2 * HT + 15) / 16 : 16;                 // M-tile bound
    constexpr int NQC = HT > 0 ? (ACC_TILES / MTC < (5 * HT + 15) / 16 ? ACC_TILES / MTC : (5 * HT + 15) / 16)
                               : ACC_TILES;                                        // N-tiles per pass bound
    const int NQ = S.Q;
    for (int pass = 0; pass < S.P; ++pass) {
        const int nbase = pass * NQ;
        f32x4 acc[MTC * NQC > ACC_TILES ? ACC_TILES : MTC * NQC];
#pragma unroll
        for (int t = 0; t < (MTC * NQC > ACC_TILES ? ACC_TILES : MTC * NQC); ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
        for (int t0 = 0; t0 < ncell; t0 += TP) {
            // cell table of the tile
            if (tid < TP) {
                const int q = t0 + tid;
                int pix = -1, flat = -1, flags = 0;
                int cst[4] = {-1, -1, -1, -1};
                if (q < ncell) {
                    const int ly = (c0 + q) / w, lx = c0 + q - ly * w;
                    pix = (y0 + ly) * D.Wc + x0 + lx;
#pragma unroll
                    for (int d = 0; d < 4; ++d) {
                        cst[d] = stash_index(h, w, ly, lx, d);
                        const bool lok = (d & 1) ? lx < w - 1 : lx > 0;   // left predecessor (y, x - sx)
                        const bool uok = (d & 2) ? ly < h - 1 : ly > 0;   // upper predecessor (y - sy, x)
                        flags |= (lok ? 1 : 0) << (2 * d) | (uok ? 2 : 0) << (2 * d);
                    }
                    const int qy = y0 + ly - ry0, qx = x0 + lx - rx0;
                    if (qy < rh && qx < rw) flat = (int)(D.flat_off[e] + qy * rw + qx);
                }
                t_pix[tid] = pix;
                t_flat[tid] = flat;
                t_flags[tid] = flags;
#pragma unroll
                for (int d = 0; d < 4; ++d) t_cst[d][tid] = cst[d];
            }
            __syncthreads();
            // issue every load of the tile, then write LDS
            float vh[MAXH], vd[MAXD], vx[MAXX];
#pragma unroll
            for (int i = 0; i < MAXH; ++i) {
                const int idx = tid + i * 256;
                int off = kOOB;
                if (idx < S.nh) {
                    const int d = idx / (TP * H2);
                    const int rem = idx - d * TP * H2;
                    const int c = rem / H2, k = rem - c * H2;
                    const int pix = t_pix[c], fl = t_flags[c] >> (2 * d);
                    const int src = k < H ? ((fl & 1) ? pix + ((d & 1) ? 1 : -1) : -1)
                                          : ((fl & 2) ? pix + ((d & 2) ? D.Wc : -D.Wc) : -1);
                    if (pix >= 0 && src >= 0) off = (d * plane + src * H + (k < H ? k : k - H)) * 4;
                }
                vh[i] = bld(rH, off);
            }
#pragma unroll
            for (int i = 0; i < MAXD; ++i) {
                const int idx = tid + i * 256;
                int off = kOOB;
                if (idx < S.nd) {
                    const int d = idx / (TP * G);
                    const int rem = idx - d * TP * G;
                    const int c = rem / G, n = rem - c * G;
                    const int cs = t_cst[d][c];
                    if (cs >= 0) {
                        const int g = n / H, k = n - g * H;  // gate, hidden unit
                        const int el = (d * (int)D.T + cell0 + cs) * H + k;
                        off = g < 4 ? el * 16 + g * 4 : (int)(z1_offset(D.T, H) * 4) + el * 4;
                    }
                }
                vd[i] = bld(rA, off);
            }
#pragma unroll
            for (int i = 0; i < MAXX; ++i) {
                const int idx = tid + i * 256;
                float v = 0.f;
                if (idx < S.nx) {
                    const int c = idx / (C + 1), r = idx - c * (C + 1);
                    const int pix = t_pix[c];
                    if (r == C) v = pix >= 0 ? 1.f : 0.f;
                    else if (pix >= 0)
                        v = BF16 ? __uint_as_float(((uint32_t)xb[(int64_t)pix * C + r]) << 16) : xf[(int64_t)pix * C + r];
                }
                vx[i] = v;
            }
#pragma unroll
            for (int i = 0; i < MAXH; ++i)
                if (tid + i * 256 < S.nh) hs[tid + i * 256] = vh[i];
#pragma unroll
            for (int i = 0; i < MAXD; ++i)
                if (tid + i * 256 < S.nd) dab[tid + i * 256] = vd[i];
#pragma unroll
            for (int i = 0; i < MAXX; ++i)
                if (tid + i * 256 < S.nx) xs[tid + i * 256] = vx[i];
            __syncthreads();
            // r^T da on the matrix cores: A = r^T (rows R, K = cells), B = da (K = cells, cols G).
            // Per k-step each M-tile's A fragment and each N-tile's B fragment is read once.
            for (int ks = 0; ks < TP; ks += 4) {
                const int c = ks + krow;
                auto a_off = [&](int mt) {
                    const int r = mt * 16 + l16;
                    return r <= C ? (int)(xs - lds) + c * (C + 1) + r
                                  : (r < R ? (int)(hs - lds) + (wd * TP + c) * H2 + (r - C - 1) : (int)(zero - lds));
                };
                auto b_off = [&](int j) {
                    const int n = (nbase + j) * 16 + l16;
                    return (n < G && j < NQ) ? (int)(dab - lds) + (wd * TP + c) * G + n : (int)(zero - lds);
                };
                if constexpr (HT > 0) {
                    float af[MTC], bf[NQC];
#pragma unroll
                    for (int mt = 0; mt < MTC; ++mt) af[mt] = mt < MT ? lds[a_off(mt)] : 0.f;
#pragma unroll
                    for (int j = 0; j < NQC; ++j) bf[j] = lds[b_off(j)];
#pragma unroll
                    for (int mt = 0; mt < MTC; ++mt)
#pragma unroll
                        for (int j = 0; j < NQC; ++j)
                            if (mt < MT && j < NQ)
                                acc[mt * NQC + j] =
                                    __builtin_amdgcn_mfma_f32_16x16x4f32(af[mt], bf[j], acc[mt * NQC + j], 0, 0, 0);
                } else {
                    // shape known only at run time: accumulator t holds M-tile t / NQ, N-tile t % NQ
#pragma unroll
                    for (int t = 0; t < ACC_TILES; ++t) {
                        const int mt = t / NQ, j = t - mt * NQ;
                        if (mt < MT)
                            acc[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(lds[a_off(mt)], lds[b_off(j)], acc[t], 0, 0, 0);
                    }
                }
            }
            if (pass == 0) {
                // dx_d = da_d Wx[d]^T for the tile's cells on the matrix cores (A = da_d: cells x G,
                // B = Wx[d]^T: G x C), per 16-cell M-tile; the four directions are then summed in order
                for (int m0 = 0; m0 < TP; m0 += 16) {
                    const bool cv = m0 + l16 < TP;       // A row = cell m0 + l16 of this tile
                    const float* arow = dab + (wd * TP + (cv ? m0 + l16 : 0)) * G;
                    for (int c0 = 0; c0 < C; c0 += 16) {
                        f32x4 dacc = f32x4{0.f, 0.f, 0.f, 0.f};
                        const int cc = c0 + l16;
#pragma unroll
                        for (int ks = 0; ks < KX; ++ks) {
                            const int n = 4 * ks + krow;
                            if (4 * ks < G) {
                                const float bv = PRE ? bwx[PRE ? ks : 0]
                                                     : ((cc < C && n < G) ? Wx[((int64_t)wd * C + cc) * G + n] : 0.f);
                                dacc = __builtin_amdgcn_mfma_f32_16x16x4f32((cv && n < G) ? arow[n] : 0.f, bv, dacc, 0, 0, 0);
                            }
                        }
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const int cell = m0 + 4 * krow + r;
                            if (cc < C && cell < TP) dxs[(wd * TP + cell) * C + cc] = dacc[r];
                        }
                    }
                }
                __syncthreads();
                for (int o = tid; o < TP * C; o += 256) {
                    const int c = o / C, chn = o - (o / C) * C;
                    if (t_pix[c] < 0) continue;
                    const float v = ((dxs[(0 * TP + c) * C + chn] + dxs[(1 * TP + c) * C + chn]) +
                                     dxs[(2 * TP + c) * C + chn]) + dxs[(3 * TP + c) * C + chn];
                    if (dx_flat && t_flat[c] >= 0) dx_flat[(int64_t)t_flat[c] * C + chn] = v;
                    if (dx_canvas) dx_canvas[(int64_t)t_pix[c] * C + chn] = t_flat[c] >= 0 ? v : 0.f;
                }
            }
            __syncthreads();
        }
        // partial sums of this segment: part[segment][d][R][G]
        float* out = part + ((int64_t)ch * 4 + wd) * R * G;
        auto store_tile = [&](int mt, int j, const f32x4& a) {
            const int col = (nbase + j) * 16 + l16;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = mt * 16 + 4 * krow + r;
                if (row < R && col < G) out[(int64_t)row * G + col] = a[r];
            }
        };
        if constexpr (HT > 0) {
#pragma unroll
            for (int mt = 0; mt < MTC; ++mt)
#pragma unroll
                for (int j = 0; j < NQC; ++j)
                    if (mt < MT && j < NQ) store_tile(mt, j, acc[mt * NQC + j]);
        } else {
#pragma unroll
            for (int t = 0; t < ACC_TILES; ++t) {
                const int mt = t / NQ, j = t - mt * NQ;
                if (mt < MT) store_tile(mt, j, acc[t]);
            }
        }
    }
}

}  // namespace

namespace {

// Partial blocks summed in a fixed order, then routed to dWx / db / dUl / dUu. A workgroup takes 64
// consecutive (direction, entry) slots (coalesced reads of each block's partial row) and 16 slices of the
// blocks: slice j adds blocks j, j + 16, j + 32, ... into four accumulators in turn, and the 16 slice sums
// are added in slice order through LDS. The loads of 16 blocks are issued before they are added, so each
// thread keeps 16 reads in flight. The order depends only on the block count, so reruns are
// bit-identical.
constexpr int RED_X = 64, RED_Y = 16, RED_U = 16;
__global__ __launch_bounds__(RED_X* RED_Y) void k_wgrad_reduce(const float* __restrict__ part, int nparts, int C,
                                                               int H, float* __restrict__ dWx,
                                                               float* __restrict__ dUl, float* __restrict__ dUu,
                                                               float* __restrict__ db) {
    const int G = 5 * H, R = C + 1 + 2 * H, E = R * G;
    const int tx = threadIdx.x % RED_X, ty = threadIdx.x / RED_X;
    const int64_t id = blockIdx.x * (int64_t)RED_X + tx;
    const bool ok = id < 4 * (int64_t)E;
    const int64_t stride = 4 * (int64_t)E;
    float s = 0.f;
    if (ok) {
        const float* p = part + id;
        float s4[4] = {0.f, 0.f, 0.f, 0.f};
        int c = ty, j = 0;
        for (; c + (RED_U - 1) * RED_Y < nparts; c += RED_U * RED_Y) {  // RED_U % 4 == 0: j is unchanged
            float v[RED_U];
#pragma unroll
            for (int u = 0; u < RED_U; ++u) v[u] = p[(int64_t)(c + u * RED_Y) * stride];
#pragma unroll
            for (int u = 0; u < RED_U; ++u) s4[u & 3] += v[u];
        }
        for (; c < nparts; c += RED_Y, j = (j + 1) & 3) s4[j] += p[(int64_t)c * stride];
        s = (s4[0] + s4[1]) + (s4[2] + s4[3]);
    }
    __shared__ float red[RED_Y][RED_X];
    red[ty][tx] = s;
    __syncthreads();
    if (ty != 0 || !ok) return;
    float t = red[0][tx];
#pragma unroll
    for (int y = 1; y < RED_Y; ++y) t += red[y][tx];
    const int d = (int)(id / E), ent = (int)(id % E);
    const int r = ent / G, n = ent % G;
    if (r < C) dWx[((int64_t)d * C + r) * G + n] = t;
    else if (r == C) db[(int64_t)d * G + n] = t;
    else if (r < C + 1 + H) dUl[((int64_t)d * H + (r - C - 1)) * G + n] = t;
    else dUu[((int64_t)d * H + (r - C - 1 - H)) * G + n] = t;
}

}  // namespace

bool wgrad_supported(int C, int H) {
    const WgradShape s = wgrad_shape(C, H);
    return s.TP * (C + 1) <= 512 && 4 * s.TP * 2 * H <= STAGE_H && 4 * s.TP * s.G <= STAGE_D && s.P <= 64 &&
           s.TP >= 4 && 5 * H <= 256 && s.MT * s.Q <= ACC_TILES;
}

size_t wgrad_lds_bytes(int C, int H) { return sizeof(float) * wgrad_lds_floats(wgrad_shape(C, H)); }

hipError_t launch_wgrad(const Dev& D, const void* x_canvas, int dtype, int C, int H, const float* h_dirs,
                        const float* dA, const float* Wx, float* part, float* dWx, float* dUl, float* dUu, float* db,
                        float* dx_flat, float* dx_canvas, hipStream_t st) {
    const WgradShape s = wgrad_shape(C, H);
    const int64_t tot = 4 * (int64_t)s.R * s.G;
    if (wgrad2_supported(C, H, dtype)) {
        hipError_t err = launch_wgrad2(D, x_canvas, dtype, C, H, h_dirs, dA, Wx, part, dx_flat, dx_canvas, st);
        if (err != hipSuccess) return err;
        launch(k_wgrad_reduce, dim3((unsigned)((tot + RED_X - 1) / RED_X)), dim3(RED_X * RED_Y), 0, st,
               part, D.ngroups, C, H, dWx, dUl, dUu, db);
        return hipGetLastError();
    }
    const size_t lds = sizeof(float) * wgrad_lds_floats(s);
    const dim3 grid((unsigned)D.nsegs), block(256);
#define MDL_WG(B, CT, HT) launch((k_wgrad_mfma<B, CT, HT>), grid, block, lds, st, D, x_canvas, s, h_dirs, \
                                 dA, Wx, part, dx_flat, dx_canvas)
    const bool bf = dtype != 0;
    if (!bf && C == 4 && H == 16) MDL_WG(false, 4, 16);
    else if (!bf && C == 1 && H == 4) MDL_WG(false, 1, 4);
    else if (bf && C == 4 && H == 32) MDL_WG(true, 4, 32);
    else if (!bf && C == 4 && H == 32) MDL_WG(false, 4, 32);
    else if (!bf && C == 4 && H == 2) MDL_WG(false, 4, 2);
    else if (!bf && C == 6 && H == 10) MDL_WG(false, 6, 10);
    else if (!bf && C == 20 && H == 50) MDL_WG(false, 20, 50);
    else if (bf) MDL_WG(true, 0, 0);
    else MDL_WG(false, 0, 0);
#undef MDL_WG
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    launch(k_wgrad_reduce, dim3((unsigned)((tot + RED_X - 1) / RED_X)), dim3(RED_X * RED_Y), 0, st, part,
           D.nsegs, C, H, dWx, dUl, dUu, db);
    return hipGetLastError();
}

}  // namespace mdl
