// k_wgrad.hip — weight and input gradients after the reverse wavefront, for any (C, H).
//
// RETURNN §4.2: after the recurrent part is back-propagated through time, the
// gradients with respect to the weights and the inputs are matrix products
// over the whole batch. For direction d, with the A-row of a computed cell p
//     r(p) = [x(p), 1, h_left(p), h_up(p)]      (C + 1 + 2H values; a predecessor
//                                              outside the example reads as zero)
// and its gate gradient da_d(p) (5H values):
//     [dWx; db; dUl; dUu][d] = sum over computed cells p of r(p)^T da_d(p)
//     dx(p)                  = sum over d of da_d(p) Wx[d]^T
// Shapes the software-pipelined kernel (k_wgrad2.hip) does not instantiate run
// here. The weight gradient is tiled like a plain GEMM whose K dimension is
// the cells of one segment of the layout's weight-gradient split: workgroup
// (segment, direction, 64 x 64 output tile) gathers r and da of 16 cells at a
// time into LDS and accumulates on v_mfma_f32_16x16x4_f32 (fp32 products and
// sums), so even a layer of few cells and many hidden units spreads over many
// workgroups. dx is a product of the same kind (canvas pixels x channels, K =
// the four directions' gate gradients) on the matrix cores. Segment
// partial sums are then added in segment order by k_wgrad_reduce, so the
// result is bit-reproducible.
#include "kernels.h"
#include "devmath.h"

namespace mdl {

WsLayout ws_layout(int64_t T, int64_t nparts, int C, int H, int64_t nflags, int64_t nfflags) {
    auto al = [](size_t v) { return (v + 255) & ~size_t(255); };
    WsLayout w;
    const int G = 5 * H;
    const int R = C + 1 + 2 * H;
    w.nparts = nparts;
    size_t p = 0;
    w.stash = p; p = al(p + sizeof(float) * 4 * (size_t)T * 8 * H);
    w.zda = p;   p = al(p + sizeof(float) * 4 * (size_t)T * G);
    w.part = p;  p = al(p + sizeof(float) * 4 * (size_t)nparts * R * G);
    w.dxp = p;   p = al(p + sizeof(float) * 4 * (size_t)T * C);
    w.flags = p; p = al(p + sizeof(int32_t) * (size_t)nflags);
    w.fflags = p; p = al(p + sizeof(int32_t) * (size_t)nfflags);
    w.total = p;
    return w;
}

namespace {

constexpr int TW_M = 64;   // output tile: rows of r^T
constexpr int TW_N = 64;   // output tile: gate columns
constexpr int TW_K = 16;   // cells staged per step
constexpr int TW_S = 80;   // LDS row stride: the four cell rows of a fragment read sit 16 banks apart

// position of region-local cell (ly, lx) of an h x w region in direction d's diagonal-major order
__device__ inline int stash_index(int h, int w, int ly, int lx, int d) {
    const int a = (d & 2) ? h - 1 - ly : ly;
    const int b = (d & 1) ? w - 1 - lx : lx;
    const int s = a + b;
    return (int)dg_start(h, w, s) + (a - dg_lo(h, w, s));
}

// grid (nsegs, 4 * MB * NB): segment; direction, M block, N block. part[segment][d][R][G].
template <bool BF16>
__global__ __launch_bounds__(256) void k_wgrad_tile(Dev D, const void* __restrict__ xc, int C, int H,
                                                    const float* __restrict__ hdirs, const float* __restrict__ dA,
                                                    float* __restrict__ part) {
    const int G = 5 * H, R = C + 1 + 2 * H;
    const int MB = (R + TW_M - 1) / TW_M, NB = (G + TW_N - 1) / TW_N;
    const int sg = blockIdx.x;
    int bz = blockIdx.y;
    const int d = bz / (MB * NB);
    bz -= d * MB * NB;
    const int mb = bz / NB, nb = bz - mb * NB;
    const int m0 = mb * TW_M, n0 = nb * TW_N;
    const int e = D.segs[3 * sg], c0 = D.segs[3 * sg + 1], c1 = D.segs[3 * sg + 2];
    const int y0 = D.rect[4 * e], x0 = D.rect[4 * e + 1], h = D.rect[4 * e + 2], w = D.rect[4 * e + 3];
    const int64_t cell0 = D.cell_off[e];
    const float* hd = hdirs + (int64_t)d * D.Hc * D.Wc * H;
    const float* dA4 = dA + (int64_t)d * D.T * 4 * H;                 // [T][H][4]: gates i, f_l, f_u, o
    const float* dA1 = dA + z1_offset(D.T, H) + (int64_t)d * D.T * H;  // [T][H]: gate g
    const float* xf = static_cast<const float*>(xc);
    const uint16_t* xb = static_cast<const uint16_t*>(xc);
    __shared__ float ra[TW_K][TW_S], da[TW_K][TW_S];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int i16 = lane & 15, q = lane >> 4;
    const int wm = (wave >> 1) * 32, wn = (wave & 1) * 32;  // this wave's 32 x 32 quarter of the tile
    f32x4 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int t0 = c0; t0 < c1; t0 += TW_K) {
        // element idx of the staged block: cell kk = idx / 64 of this step, tile column col = idx % 64
#pragma unroll
        for (int it = 0; it < TW_K * 64 / 256; ++it) {
            const int idx = tid + 256 * it;
            const int kk = idx >> 6, col = idx & 63;
            const int cq = t0 + kk;
            float rv = 0.f, dv = 0.f;
            if (cq < c1) {
                const int ly = cq / w, lx = cq - ly * w;
                const int pix = (y0 + ly) * D.Wc + x0 + lx;
                const int ri = m0 + col;
                if (ri < C) {
                    rv = BF16 ? __uint_as_float((uint32_t)xb[(int64_t)pix * C + ri] << 16) : xf[(int64_t)pix * C + ri];
                } else if (ri == C) {
                    rv = 1.f;
                } else if (ri < C + 1 + H) {  // left predecessor (y, x - sx)
                    if ((d & 1) ? lx < w - 1 : lx > 0) rv = hd[(int64_t)(pix + ((d & 1) ? 1 : -1)) * H + (ri - C - 1)];
                } else if (ri < R) {          // upper predecessor (y - sy, x)
                    if ((d & 2) ? ly < h - 1 : ly > 0)
                        rv = hd[(int64_t)(pix + ((d & 2) ? D.Wc : -D.Wc)) * H + (ri - C - 1 - H)];
                }
                const int n = n0 + col;
                if (n < G) {
                    const int g = n / H, k = n - g * H;
                    const int64_t t = cell0 + stash_index(h, w, ly, lx, d);
                    dv = g < 4 ? dA4[(t * H + k) * 4 + g] : dA1[t * H + k];
                }
            }
            ra[kk][col] = rv;
            da[kk][col] = dv;
        }
        __syncthreads();
#pragma unroll
        for (int ks = 0; ks < TW_K / 4; ++ks) {
            const int c = 4 * ks + q;  // lane (q, i16) supplies A[i16][q] = r(cell c)[row] and B[q][i16]
            const float a0 = ra[c][wm + i16], a1 = ra[c][wm + 16 + i16];
            const float b0 = da[c][wn + i16], b1 = da[c][wn + 16 + i16];
            acc[0][0] = __builtin_amdgcn_mfma_f32_16x16x4f32(a0, b0, acc[0][0], 0, 0, 0);
            acc[0][1] = __builtin_amdgcn_mfma_f32_16x16x4f32(a0, b1, acc[0][1], 0, 0, 0);
            acc[1][0] = __builtin_amdgcn_mfma_f32_16x16x4f32(a1, b0, acc[1][0], 0, 0, 0);
            acc[1][1] = __builtin_amdgcn_mfma_f32_16x16x4f32(a1, b1, acc[1][1], 0, 0, 0);
        }
        __syncthreads();
    }
    float* out = part + ((int64_t)sg * 4 + d) * R * G;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = m0 + wm + 16 * i + 4 * q + r, col = n0 + wn + 16 * j + i16;
                if (row < R && col < G) out[(int64_t)row * G + col] = acc[i][j][r];
            }
}

// dx(p)[c] = sum over d (in order 0..3) of da_d(p) . Wx[d][c][:], written for computed cells: dx_flat at
// the real pixels, dx_canvas at every computed cell (zero outside the real pixels). A workgroup takes 16
// canvas pixels (one MFMA row tile), wave d direction d: v_mfma_f32_16x16x4_f32 with A = the pixels' gate
// gradients (K: first the 4H values (unit, gate < 4) in their stored order, then the H values of gate 4)
// and B = Wx[d] in the same K order, 16 channels at a time; the four directions are added through LDS.
constexpr int DX_PIX = 16;
__global__ __launch_bounds__(256) void k_dx_cells(Dev D, int C, int H, const float* __restrict__ dA,
                                                  const float* __restrict__ Wx, float* __restrict__ dx_flat,
                                                  float* __restrict__ dx_canvas) {
    const int G = 5 * H;
    const int lane = threadIdx.x & 63, d = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int i16 = lane & 15, q = lane >> 4;
    const int64_t P = (int64_t)D.Hc * D.Wc;
    const int64_t p0 = (int64_t)blockIdx.x * DX_PIX;
    // this lane's A row: pixel p0 + i16
    const int64_t pa = p0 + i16;
    const int ea = pa < P ? D.eid[pa] : -1;
    const float* a4 = dA;  // [4H] of the pixel's cell in direction d
    const float* a1 = dA;  // [H]
    if (ea >= 0) {
        const int y0 = D.rect[4 * ea], x0 = D.rect[4 * ea + 1], h = D.rect[4 * ea + 2], w = D.rect[4 * ea + 3];
        const int ly = (int)(pa / D.Wc) - y0, lx = (int)(pa % D.Wc) - x0;
        const int64_t t = (int64_t)d * D.T + D.cell_off[ea] + stash_index(h, w, ly, lx, d);
        a4 = dA + t * 4 * H;
        a1 = dA + z1_offset(D.T, H) + t * H;
    }
    __shared__ float red[4][DX_PIX][17];
    for (int cb = 0; cb < C; cb += 16) {
        const int c = cb + i16;  // this lane's B column
        const bool cok = c < C;
        const float* wr = Wx + ((int64_t)d * C + (cok ? c : 0)) * G;
        f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
        for (int ks = 0; ks < H; ++ks) {  // K index 4 ks + q: unit ks, gate q
            const float av = ea >= 0 ? a4[4 * ks + q] : 0.f;
            const float bv = cok ? wr[q * H + ks] : 0.f;
            acc = __builtin_amdgcn_mfma_f32_16x16x4f32(av, bv, acc, 0, 0, 0);
        }
        for (int ks = 0; 4 * ks < H; ++ks) {  // gate 4 of unit 4 ks + q
            const int k = 4 * ks + q;
            const float av = (ea >= 0 && k < H) ? a1[k] : 0.f;
            const float bv = (cok && k < H) ? wr[4 * H + k] : 0.f;
            acc = __builtin_amdgcn_mfma_f32_16x16x4f32(av, bv, acc, 0, 0, 0);
        }
        __syncthreads();  // the previous block's sums have been read
#pragma unroll
        for (int r = 0; r < 4; ++r) red[d][4 * q + r][i16] = acc[r];  // pixel row 4q + r, channel column i16
        __syncthreads();
        const int pr = threadIdx.x >> 4, cc = threadIdx.x & 15;
        const int64_t pix = p0 + pr;
        if (pr < DX_PIX && pix < P && cb + cc < C) {
            const int e = D.eid[pix];
            if (e >= 0) {
                const float v = ((red[0][pr][cc] + red[1][pr][cc]) + red[2][pr][cc]) + red[3][pr][cc];
                const int qy = (int)(pix / D.Wc) - D.real[4 * e], qx = (int)(pix % D.Wc) - D.real[4 * e + 1];
                const bool real = qy < D.real[4 * e + 2] && qx < D.real[4 * e + 3];
                if (dx_flat && real)
                    dx_flat[(D.flat_off[e] + (int64_t)qy * D.real[4 * e + 3] + qx) * C + cb + cc] = v;
                if (dx_canvas) dx_canvas[pix * C + cb + cc] = real ? v : 0.f;
            }
        }
    }
}

}  // namespace

namespace {

// Partial blocks summed in a fixed order, then routed to dWx / db / dUl / dUu. A workgroup takes 64
// consecutive (direction, entry) slots (coalesced reads of each block's partial row) and RY slices of the
// blocks: slice j adds blocks j, j + RY, j + 2 RY, ... into four accumulators in turn, and the RY slice sums
// are added in slice order through LDS. The loads of 16 blocks are issued before they are added (a missing
// block reads as zero), so each thread keeps 16 reads in flight. RY is 16 for many blocks and 4 for few
// (at most 64), so that a few blocks still fill the loads of one round. The order depends only on the
// block count, so reruns are bit-identical.
constexpr int RED_X = 64, RED_U = 16;
template <int RY>
__global__ __launch_bounds__(RED_X* RY) void k_wgrad_reduce(const float* __restrict__ part, int nparts, int C, int H,
                                                            float* __restrict__ dWx, float* __restrict__ dUl,
                                                            float* __restrict__ dUu, float* __restrict__ db) {
    const int G = 5 * H, R = C + 1 + 2 * H, E = R * G;
    const int tx = threadIdx.x % RED_X, ty = threadIdx.x / RED_X;
    const int64_t id = blockIdx.x * (int64_t)RED_X + tx;
    const bool ok = id < 4 * (int64_t)E;
    const int64_t stride = 4 * (int64_t)E;
    float s = 0.f;
    if (ok) {
        const float* p = part + id;
        float s4[4] = {0.f, 0.f, 0.f, 0.f};
        for (int c = ty; c < nparts; c += RED_U * RY) {
            float v[RED_U];
#pragma unroll
            for (int u = 0; u < RED_U; ++u) v[u] = c + u * RY < nparts ? p[(int64_t)(c + u * RY) * stride] : 0.f;
#pragma unroll
            for (int u = 0; u < RED_U; ++u) s4[u & 3] += v[u];
        }
        s = (s4[0] + s4[1]) + (s4[2] + s4[3]);
    }
    __shared__ float red[RY][RED_X];
    red[ty][tx] = s;
    __syncthreads();
    if (ty != 0 || !ok) return;
    float t = red[0][tx];
#pragma unroll
    for (int y = 1; y < RY; ++y) t += red[y][tx];
    const int d = (int)(id / E), ent = (int)(id % E);
    const int r = ent / G, n = ent % G;
    if (r < C) dWx[((int64_t)d * C + r) * G + n] = t;
    else if (r == C) db[(int64_t)d * G + n] = t;
    else if (r < C + 1 + H) dUl[((int64_t)d * H + (r - C - 1)) * G + n] = t;
    else dUu[((int64_t)d * H + (r - C - 1 - H)) * G + n] = t;
}

}  // namespace

size_t wgrad_lds_bytes(int, int) { return 2 * sizeof(float) * TW_K * TW_S; }

hipError_t launch_wgrad_reduce(int64_t nparts, int C, int H, const float* part, float* dWx, float* dUl, float* dUu,
                               float* db, hipStream_t st) {
    const int G = 5 * H, R = C + 1 + 2 * H;
    const int64_t tot = 4 * (int64_t)R * G;
    const dim3 rgrid((unsigned)((tot + RED_X - 1) / RED_X));
    if (nparts > 64)
        launch(k_wgrad_reduce<16>, rgrid, dim3(RED_X * 16), 0, st, part, (int)nparts, C, H, dWx, dUl, dUu, db);
    else
        launch(k_wgrad_reduce<4>, rgrid, dim3(RED_X * 4), 0, st, part, (int)nparts, C, H, dWx, dUl, dUu, db);
    return hipGetLastError();
}

hipError_t launch_wgrad(const Dev& D, const void* x_canvas, int dtype, int C, int H, const float* h_dirs,
                        const float* dA, const float* Wx, float* part, float* dxp, float* dWx, float* dUl, float* dUu,
                        float* db, float* dx_flat, float* dx_canvas, hipStream_t st) {
    const int G = 5 * H, R = C + 1 + 2 * H;
    int64_t nparts = D.ngroups;
    if (wgrad2_supported(C, H, dtype)) {
        const bool want_dx = dx_flat != nullptr || dx_canvas != nullptr;
        hipError_t err = launch_wgrad2(D, x_canvas, dtype, C, H, h_dirs, dA, Wx, part, want_dx ? dxp : nullptr, st);
        if (err == hipSuccess) err = launch_dx_sum(D, C, dxp, dx_flat, dx_canvas, st);
        if (err != hipSuccess) return err;
    } else {
        const int MB = (R + TW_M - 1) / TW_M, NB = (G + TW_N - 1) / TW_N;
        const dim3 grid((unsigned)D.nsegs, (unsigned)(4 * MB * NB));
        if (dtype != 0) launch(k_wgrad_tile<true>, grid, dim3(256), 0, st, D, x_canvas, C, H, h_dirs, dA, part);
        else launch(k_wgrad_tile<false>, grid, dim3(256), 0, st, D, x_canvas, C, H, h_dirs, dA, part);
        hipError_t err = hipGetLastError();
        if (err != hipSuccess) return err;
        if (dx_flat || dx_canvas) {
            const int64_t P = (int64_t)D.Hc * D.Wc;
            launch(k_dx_cells, dim3((unsigned)((P + DX_PIX - 1) / DX_PIX)), dim3(256), 0, st, D, C, H, dA, Wx,
                   dx_flat, dx_canvas);
            err = hipGetLastError();
            if (err != hipSuccess) return err;
        }
        nparts = D.nsegs;
    }
    return launch_wgrad_reduce(nparts, C, H, part, dWx, dUl, dUu, db, st);
}

}  // namespace mdl
