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
#include "devmath.h"

namespace mdl {

namespace {

constexpr int CHAIN_THREADS = 256;
constexpr int MAXI = 8;  // (cell, hidden) items per thread and step

// Forward. Z in (Z4, Z1), the forward values the reverse wavefront needs out (SA, SB), h_dirs out [4][Hc][Wc][H].
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
    const float* Z4d = Z + base * 4 * H;
    const float* Z1d = Z + z1_offset(D.T, H) + base * H;
    float* S4d = stash + base * 4 * H;
    float* SBd = stash + z1_offset(D.T, H) + base * 4 * H;
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
                for (int g = 0; g < 4; ++g) zc[i][g] = Z4d[((int64_t)j * H + k) * 4 + g];
                zc[i][4] = Z1d[(int64_t)j * H + k];
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
                    for (int g = 0; g < 4; ++g) zn[i][g] = Z4d[((stn + j) * H + k) * 4 + g];
                    zn[i][4] = Z1d[(stn + j) * H + k];
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
                const float gg = ftanh(acc4);
                const float c = fl * cl + fu * cu + ig * gg;
                const float tc = ftanh(c);
                const float hv = og * tc;
                hn[j * H + k] = hv;
                cn[j * H + k] = c;
                Hd[((int64_t)F.y(a) * D.Wc + F.x(b)) * H + k] = hv;
                *reinterpret_cast<f32x4*>(S4d + ((st + j) * H + k) * 4) = f32x4{ig, fl, fu, og};
                *reinterpret_cast<f32x4*>(SBd + ((st + j) * H + k) * 4) = f32x4{gg, tc, cl, cu};
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
// for every direction) or dh_dirs [4][Hc][Wc][H]. dA out (dA4, dA1).
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
    const float* SAd = stash + base * 4 * H;
    const float* SBd = stash + z1_offset(D.T, H) + base * 4 * H;
    float* dA4d = dA + base * 4 * H;
    float* dA1d = dA + z1_offset(D.T, H) + base * H;
    const float* dyb = dy_flat ? dy_flat + D.flat_off[e] * H : nullptr;
    const float* dhd = dh_dirs ? dh_dirs + (int64_t)d * D.Hc * D.Wc * H : nullptr;
    const int S = h + w - 1;
    const int tid = threadIdx.x, nthr = blockDim.x;

    for (int s = S - 1; s >= 0; --s) {
        const int L = dg_len(h, w, s), lo = dg_lo(h, w, s);
        const int64_t st = dg_start(h, w, s);
        const int lon = dg_lo(h, w, s + 1);
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
                // the forward's values of this cell, and the factors from them
                f32x4 fa, fb;
                bwd_factors(*reinterpret_cast<const f32x4*>(SAd + ((st + j) * H + k) * 4),
                            *reinterpret_cast<const f32x4*>(SBd + ((st + j) * H + k) * 4), fa, fb);
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
                const float dc = __builtin_fmaf(dh, fb[1], dcin);
                const float d0 = dc * fa[0], d1 = dc * fa[1], d2 = dc * fa[2], d3 = dh * fa[3], d4 = dc * fb[0];
                float* dw = daw + j * G + k;
                dw[0] = d0; dw[H] = d1; dw[2 * H] = d2; dw[3 * H] = d3; dw[4 * H] = d4;
                dclw[j * H + k] = dc * fb[2];
                dcuw[j * H + k] = dc * fb[3];
                float* dg = dA4d + ((st + j) * H + k) * 4;
                dg[0] = d0; dg[1] = d1; dg[2] = d2; dg[3] = d3;
                dA1d[(st + j) * H + k] = d4;
            }
        }
        __syncthreads();
    }
}


// ---------------------------------------------------------------------------------------------
// Matrix-core variants. The recurrent contraction of one step is dense: for the
// cells of a diagonal, [h_left | h_up] (2H) times [Ul; Uu] (2H x 5H) in the
// forward, [da_right | da_down] (10H) times [Ul^T; Uu^T] (10H x H) in the
// backward. Each wave owns one block of 16 hidden units (kb) and keeps that
// block's weight columns as v_mfma_f32_16x16x4_f32 B fragments in registers
// for the whole pass; the A fragments (16 cells x 4 inputs) come from the LDS
// copy of the previous diagonal, with a zero row standing in for predecessors
// outside the example. Gate columns are taken per gate type for the lane's
// hidden unit, so after the MFMAs each lane holds all five pre-activations of
// its 4 (cell, hidden unit) pairs and finishes the cell update in registers.
// The projection x.Wx+b seeds the accumulators; next-step operands are
// prefetched from HBM while the current step computes.
// ---------------------------------------------------------------------------------------------

// All global traffic of the step loops goes through raw buffer loads/stores
// (devmath.h); kOOB is an offset past every per-unit range used here (1 GiB).
constexpr int kOOB = 0x40000000;

template <int H>
__global__ __launch_bounds__(256) void k_bwd_mfma(Dev D, int, int Lmax, const float* __restrict__ Ul,
                                                  const float* __restrict__ Uu, const float* __restrict__ stash,
                                                  const float* __restrict__ dy_flat,
                                                  const float* __restrict__ dh_dirs, float* __restrict__ dA) {
    constexpr int G = 5 * H;
    constexpr int KS = (2 * G + 3) / 4;        // k-steps over [da_right; da_down]
    constexpr int KB = H <= 16 ? 1 : H <= 32 ? 2 : 4;
    const int u = D.units[blockIdx.x];
    const int e = u >> 2, d = u & 3;
    const Flip F{D.rect[4 * e], D.rect[4 * e + 1], D.rect[4 * e + 2], D.rect[4 * e + 3], (d & 2) != 0, (d & 1) != 0};
    const int h = F.h, w = F.w;
    const int ry0 = D.real[4 * e], rx0 = D.real[4 * e + 1], rh = D.real[4 * e + 2], rw = D.real[4 * e + 3];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int kb = wave % KB, mt = wave / KB;
    const int kk = kb * 16 + (lane & 15);
    const bool kok = kk < H;
    const int krow = lane >> 4;
    const int orow = mt * 16 + 4 * (lane >> 4);

    float Bw[KS];                               // [Ul^T; Uu^T][4ks + krow][kk]
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        const int n = 4 * ks + krow;
        float v = 0.f;
        if (kok && n < 2 * G)
            v = n < G ? Ul[((int64_t)d * H + kk) * G + n] : Uu[((int64_t)d * H + kk) * G + n - G];
        Bw[ks] = v;
    }
    extern __shared__ float lds[];
    const int ZR = 16 * ((Lmax + 15) / 16);
    const int LR = ZR + 1;
    float* dab = lds;                           // [2][LR][G]   gate gradients of the later diagonal
    float* dcl = dab + 2 * LR * G;              // [2][LR][H]   dc * f_l
    float* dcu = dcl + 2 * LR * H;              // [2][LR][H]   dc * f_u
    for (int i = threadIdx.x; i < 2 * LR * G + 4 * LR * H; i += blockDim.x) lds[i] = 0.f;
    const int64_t base = (int64_t)d * D.T + D.cell_off[e];
    const int64_t cells = (int64_t)h * w;
    const __amdgpu_buffer_rsrc_t rS4 = rsrc(stash + base * 4 * H, cells * 4 * H * 4);
    const __amdgpu_buffer_rsrc_t rS2 = rsrc(stash + z1_offset(D.T, H) + base * 4 * H, cells * 4 * H * 4);
    const __amdgpu_buffer_rsrc_t rA4 = rsrc(dA + base * 4 * H, cells * 16 * H);
    const __amdgpu_buffer_rsrc_t rA1 = rsrc(dA + z1_offset(D.T, H) + base * H, cells * 4 * H);
    // upstream gradient: per-direction canvas tensor, or the flat gradient of the direction sum
    const bool per_dir = dh_dirs != nullptr;
    const __amdgpu_buffer_rsrc_t rU =
        per_dir ? rsrc(dh_dirs + (int64_t)d * D.Hc * D.Wc * H, (int64_t)D.Hc * D.Wc * H * 4)
                : rsrc(dy_flat + D.flat_off[e] * H, (int64_t)rh * rw * H * 4);
    const int S = h + w - 1;

    // per output cell: the forward's values (SA 0-3, SB 4-7), upstream dh
    auto load_v = [&](int s, float (&v)[9][4]) {
        const bool in = s >= 0;
        const int L = in ? dg_len(h, w, s) : 0, lo = in ? dg_lo(h, w, s) : 0;
        const int st = in ? (int)dg_start(h, w, s) : 0;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int jo = orow + r;
            const bool ok = jo < L && kok;
            const int a = lo + jo, b = s - a;
            const int ei = (st + jo) * H + kk;  // (cell, hidden unit) element of the stash
            const int so = ok ? ei * 16 : kOOB;
#pragma unroll
            for (int g = 0; g < 4; ++g) v[g][r] = bld(rS4, so + g * 4);
#pragma unroll
            for (int g = 0; g < 4; ++g) v[4 + g][r] = bld(rS2, so + g * 4);
            const int y = F.y(a), x = F.x(b);
            const int ly = y - ry0, lx = x - rx0;
            int uo = kOOB;
            if (ok && per_dir) uo = (int)(((int64_t)y * D.Wc + x) * H + kk) * 4;
            if (ok && !per_dir && ly < rh && lx < rw) uo = ((ly * rw + lx) * H + kk) * 4;
            v[8][r] = bld(rU, uo);
        }
    };
    auto step = [&](int s, float (&vc)[9][4], float (&vn)[9][4]) {
        const int L = dg_len(h, w, s), lo = dg_lo(h, w, s);
        const int st = (int)dg_start(h, w, s);
        const int lon = dg_lo(h, w, s + 1);
        load_v(s - 1, vn);                      // prefetch; consumed one step later
        const float* dar = dab + ((s + 1) & 1) * LR * G;
        const float* dclr = dcl + ((s + 1) & 1) * LR * H;
        const float* dcur = dcu + ((s + 1) & 1) * LR * H;
        float* daw = dab + (s & 1) * LR * G;
        float* dclw = dcl + (s & 1) * LR * H;
        float* dcuw = dcu + (s & 1) * LR * H;
        f32x4 acc = f32x4{vc[8][0], vc[8][1], vc[8][2], vc[8][3]};
        if (mt * 16 < L) {                      // uniform over the wave; no global memory inside
            const int ja = mt * 16 + (lane & 15);
            const int aA = lo + ja, bA = s - aA;
            const int jr = (ja < L && bA + 1 < w) ? aA - lon : ZR;       // right successor (a, b+1)
            const int jd = (ja < L && aA + 1 < h) ? aA + 1 - lon : ZR;   // lower successor (a+1, b)
            // A operand addresses first (zero row for a missing successor), one unconditional LDS read
            // per k-step issued ahead of the MFMAs; two accumulators halve the dependent chain
            float av[KS];
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const int n = 4 * ks + krow;
                const int idx = n < G ? jr * G + n : (n < 2 * G ? jd * G + n - G : ZR * G);
                av[ks] = dar[idx];
            }
            f32x4 acc2 = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                if (ks & 1) acc2 = __builtin_amdgcn_mfma_f32_16x16x4f32(av[ks], Bw[ks], acc2, 0, 0, 0);
                else acc = __builtin_amdgcn_mfma_f32_16x16x4f32(av[ks], Bw[ks], acc, 0, 0, 0);
            }
            acc += acc2;
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int jo = orow + r;
            const bool ok = jo < L && kok;
            const int a = lo + jo, b = s - a;
            const float dh = acc[r];
            const int kc = kok ? kk : 0;
            const float dcin = dclr[((ok && b + 1 < w) ? a - lon : ZR) * H + kc] +
                               dcur[((ok && a + 1 < h) ? a + 1 - lon : ZR) * H + kc];
            f32x4 ka, kb;
            bwd_factors(f32x4{vc[0][r], vc[1][r], vc[2][r], vc[3][r]}, f32x4{vc[4][r], vc[5][r], vc[6][r], vc[7][r]},
                        ka, kb);
            const float dc = __builtin_fmaf(dh, kb[1], dcin);
            const float d0 = dc * ka[0], d1 = dc * ka[1], d2 = dc * ka[2], d3 = dh * ka[3], d4 = dc * kb[0];
            if (ok) {
                float* dw = daw + jo * G + kk;
                dw[0] = d0; dw[H] = d1; dw[2 * H] = d2; dw[3 * H] = d3; dw[4 * H] = d4;
                dclw[jo * H + kk] = dc * kb[2];
                dcuw[jo * H + kk] = dc * kb[3];
            }
            const int ea = (st + jo) * H + kk;
            const int a4 = ok ? ea * 16 : kOOB, a1 = ok ? ea * 4 : kOOB;
            bst(d0, rA4, a4);
            bst(d1, rA4, a4 + 4);
            bst(d2, rA4, a4 + 8);
            bst(d3, rA4, a4 + 12);
            bst(d4, rA1, a1);
        }
        __syncthreads();
    };
    float vA[9][4], vB[9][4];
    load_v(S - 1, vA);
    __syncthreads();
    int s = S - 1;
    for (; s - 1 >= 0; s -= 2) {
        step(s, vA, vB);
        step(s - 1, vB, vA);
    }
    if (s >= 0) step(s, vA, vB);
}

typedef void (*BwdKernel)(Dev, int, int, const float*, const float*, const float*, const float*, const float*, float*);

// instantiated hidden sizes: the workloads' 2, 4, 10, 16, 32 and 50
struct MfmaEntry {
    int H;
    BwdKernel bwd;
    int KB;
};
// hidden sizes with a vector-ALU or f16 reverse wavefront take those over the diagonal widths they cover
const MfmaEntry kMfma[] = {
    {50, k_bwd_mfma<50>, 4},
};

// one M-tile of 16 cells per wave: 4/KB tiles cover the widest diagonal
const MfmaEntry* mfma_entry(int H, int Lmax) {
    for (const auto& m : kMfma)
        if (m.H == H) return (Lmax + 15) / 16 <= 4 / m.KB ? &m : nullptr;
    return nullptr;
}

int lds_rows(int Lmax) { return 16 * ((Lmax + 15) / 16) + 1; }
size_t bwd_mfma_lds(int H, int Lmax) {
    return sizeof(float) * ((size_t)2 * lds_rows(Lmax) * 5 * H + (size_t)4 * lds_rows(Lmax) * H);
}

}  // namespace

int chain_max_items() { return MAXI * CHAIN_THREADS; }


size_t fwd_chain_lds(int H, int Lmax) {
    return sizeof(float) * ((size_t)2 * H * 5 * H + (size_t)4 * Lmax * H);
}

size_t bwd_chain_lds(int H, int Lmax) {
    if (small_bwd_supported(H, Lmax)) return small_bwd_lds(H, Lmax);
    if (bwd16_supported(H, Lmax)) return bwd16_lds(H, Lmax);
    if (mfma_entry(H, Lmax)) return bwd_mfma_lds(H, Lmax);
    return sizeof(float) * ((size_t)2 * H * 5 * H + (size_t)2 * Lmax * 5 * H + (size_t)4 * Lmax * H);
}

bool chain_uses_mfma(int H, int Lmax) { return mfma_entry(H, Lmax) != nullptr; }

hipError_t launch_fwd_chain(const Dev& D, int H, const float* Ul, const float* Uu, const float* Z, float* stash,
                            float* h_dirs, hipStream_t st) {
    const int Lmax = D.max_diag;
    launch(k_fwd_chain, dim3(4 * D.n), dim3(CHAIN_THREADS), fwd_chain_lds(H, Lmax), st, D, H, Lmax, Ul,
           Uu, Z, stash, h_dirs);
    return hipGetLastError();
}

hipError_t launch_bwd_chain(const Dev& D, int H, const float* Ul, const float* Uu, const float* stash,
                            const float* dy_flat, const float* dh_dirs, float* dA, hipStream_t st) {
    const int Lmax = D.max_diag;
    if (small_bwd_supported(H, Lmax)) return launch_bwd_small(D, H, Ul, Uu, stash, dy_flat, dh_dirs, dA, st);
    if (bwd16_supported(H, Lmax)) return launch_bwd16(D, H, Ul, Uu, stash, dy_flat, dh_dirs, dA, nullptr, st);
    if (const MfmaEntry* m = mfma_entry(H, Lmax)) {
        launch(m->bwd, dim3(4 * D.n), dim3(256), bwd_mfma_lds(H, Lmax), st, D, H, Lmax, Ul, Uu, stash,
               dy_flat, dh_dirs, dA);
        return hipGetLastError();
    }
    launch(k_bwd_chain, dim3(4 * D.n), dim3(CHAIN_THREADS), bwd_chain_lds(H, Lmax), st, D, H, Lmax, Ul,
           Uu, stash, dy_flat, dh_dirs, dA);
    return hipGetLastError();
}

}  // namespace mdl
