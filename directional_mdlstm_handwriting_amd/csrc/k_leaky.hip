// k_leaky.hip — the Leaky-LP cell ("No Padding Please" §III, Figure 4(b); §IX-A): forward and reverse
// wavefronts on the fp32 matrix cores, and the weight gradients of its memory-state projections.
//
// The cell, per direction and hidden unit, with the predecessors' (h, s) read as (0, 0) outside the example:
//     a    = x.Wx + b + h_l.Ul + h_u.Uu                (5H: f, lam, o1, o2, g)
//     a[lam, o1, o2] += s_l.Vl + s_u.Vu                (3H: the memory-state projections)
//     sbar = lam s_l + (1 - lam) s_u                   (lambda gate: a convex combination)
//     s    = f sbar + (1 - f) g                        (leaky update: a convex combination)
//     h    = o1 tanh(s) + o2 s                         (two output gates)
// The schedule is that of the other wavefront kernels: one workgroup per (example, direction) unit walks its
// local anti-diagonals (all cells of one are independent). Wave (tile mt, block kb) owns 16 cells of the
// diagonal (MFMA rows) and 16 hidden units (MFMA columns); its weight columns sit in registers as
// v_mfma_f32_16x16x4_f32 B fragments for the whole pass, the previous diagonal's h and s (forward) or gate
// gradients (backward) in LDS ping-pong buffers, with a zero row standing in for a missing neighbour. Every
// product is an fp32 product: the recurrence needs no operand splitting here.
//
// The forward stash keeps the layout of the plain cell's, six values per (cell, hidden unit): (f, lam, o1,
// o2) then (g, s); the gate gradients dA likewise: (f, lam, o1, o2) then g. So the weight gradients of Wx,
// b, Ul, Uu and the input gradient are those of the plain cell's kernels (their inputs are the same); only
// dVl and dVu are computed here, from the stash's memory states and the lam, o1, o2 columns of dA.
#include "kernels.h"
#include "devmath.h"
#include "leaky16.h"

namespace mdl {

namespace {

constexpr int kOOBl = 0x40000000;  // byte offset past every per-unit range used here (1 GiB)
constexpr int kMaxKX = 4;          // input channels up to 16

template <int H>
struct LeakyShape {
    static constexpr int NB = (H + 15) / 16;  // 16-wide blocks of hidden units
    static constexpr int KP = (2 * H + 3) / 4;  // k-steps over a predecessor pair [left | up] of H values each
    static constexpr int RS = 2 * H + 4;        // LDS row of the forward: h then s; stride 4 mod 32 words
    static constexpr int RG = 5 * H + 4;        // LDS row of the backward: the five gate gradients
    static constexpr int RD = H + 4;            // LDS row of the backward: ds sent to a predecessor
    // threads per workgroup at most: with two blocks of hidden units the weight fragments need the whole
    // register file of a SIMD (one wave per SIMD), with one block two waves per SIMD fit
    static constexpr int MAXT = NB >= 2 ? 256 : 512;
};

// Forward. XBF: canvas pixels stored as bf16.
template <int H, bool XBF>
__global__ __launch_bounds__(LeakyShape<H>::MAXT) void k_fwd_leaky(Dev D, const void* __restrict__ xc, int C, int NT,
                                                    const float* __restrict__ Wx, const float* __restrict__ bias,
                                                    const float* __restrict__ Ul, const float* __restrict__ Uu,
                                                    const float* __restrict__ Vl, const float* __restrict__ Vu,
                                                    float* __restrict__ stash, float* __restrict__ hdirs) {
    using Sh = LeakyShape<H>;
    constexpr int NB = Sh::NB, KP = Sh::KP, RS = Sh::RS, G = 5 * H, G3 = 3 * H;
    const int u = D.units[blockIdx.x];
    const int e = u >> 2, d = u & 3;
    const Flip F{D.rect[4 * e], D.rect[4 * e + 1], D.rect[4 * e + 2], D.rect[4 * e + 3], (d & 2) != 0, (d & 1) != 0};
    const int h = F.h, w = F.w;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int mt = wave / NB, kb = wave % NB;
    const int col = lane & 15, krow = lane >> 4;
    const int kk = kb * 16 + col;
    const bool kok = kk < H;
    const int KX = (C + 3) / 4;

    // B fragments: lane holds row 4 ks + krow, column kk of each gate's weights
    float Bh[5][KP], Bs[3][KP], Bx[5][kMaxKX], bz[5];
#pragma unroll
    for (int g = 0; g < 5; ++g) {
        bz[g] = kok ? bias[(int64_t)d * G + g * H + kk] : 0.f;
#pragma unroll
        for (int ks = 0; ks < KP; ++ks) {
            const int n = 4 * ks + krow;
            float v = 0.f;
            if (kok && n < H) v = Ul[((int64_t)d * H + n) * G + g * H + kk];
            else if (kok && n < 2 * H) v = Uu[((int64_t)d * H + n - H) * G + g * H + kk];
            Bh[g][ks] = v;
        }
#pragma unroll
        for (int ks = 0; ks < kMaxKX; ++ks) {
            const int c = 4 * ks + krow;
            Bx[g][ks] = (kok && ks < KX && c < C) ? Wx[((int64_t)d * C + c) * G + g * H + kk] : 0.f;
        }
    }
#pragma unroll
    for (int m = 0; m < 3; ++m)
#pragma unroll
        for (int ks = 0; ks < KP; ++ks) {
            const int n = 4 * ks + krow;
            float v = 0.f;
            if (kok && n < H) v = Vl[((int64_t)d * H + n) * G3 + m * H + kk];
            else if (kok && n < 2 * H) v = Vu[((int64_t)d * H + n - H) * G3 + m * H + kk];
            Bs[m][ks] = v;
        }

    extern __shared__ __align__(16) float lds[];
    const int ZR = 16 * NT, ROWS = ZR + 1;
    for (int i = threadIdx.x; i < 2 * ROWS * RS; i += blockDim.x) lds[i] = 0.f;

    const int64_t base = (int64_t)d * D.T + D.cell_off[e];
    const int64_t cells = (int64_t)h * w;
    const int XB = XBF ? 2 : 4;
    const __amdgpu_buffer_rsrc_t rX = rsrc(xc, (int64_t)D.Hc * D.Wc * C * XB);
    const __amdgpu_buffer_rsrc_t rS4 = rsrc(stash + base * 4 * H, cells * 16 * H);
    const __amdgpu_buffer_rsrc_t rS2 = rsrc(stash + z1_offset(D.T, H) + base * 2 * H, cells * 8 * H);
    const __amdgpu_buffer_rsrc_t rH = rsrc(hdirs + (int64_t)d * D.Hc * D.Wc * H, (int64_t)D.Hc * D.Wc * H * 4);
    const int S = h + w - 1;
    const int ja = mt * 16 + col;  // this lane's A row: its cell on the diagonal

    // input pixels of the A row's cell on diagonal s1, one value per k-step of channels (0 where absent)
    auto load_x = [&](int s1, float (&xv)[kMaxKX]) {
        const bool in = s1 < S;
        const int L1 = in ? dg_len(h, w, s1) : 0, lo1 = in ? dg_lo(h, w, s1) : 0;
        const int a = lo1 + ja, b = s1 - a;
        const bool va = ja < L1;
        const int px = va ? F.y(a) * D.Wc + F.x(b) : 0;
#pragma unroll
        for (int ks = 0; ks < kMaxKX; ++ks) {
            const int c = 4 * ks + krow;
            const int off = (va && ks < KX && c < C) ? (px * C + c) * XB : kOOBl;
            if constexpr (XBF)
                xv[ks] = __uint_as_float((uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rX, off, 0, 0) << 16);
            else
                xv[ks] = bld(rX, off);
        }
    };
    float xa[kMaxKX], xb[kMaxKX];
    load_x(0, xa);
    __syncthreads();

    auto step = [&](int s, const float (&xv)[kMaxKX], float (&xn)[kMaxKX]) {
        const int L = dg_len(h, w, s), lo = dg_lo(h, w, s);
        const int st = (int)dg_start(h, w, s);
        const int dl = s > 0 ? lo - dg_lo(h, w, s - 1) : 0;  // position shift to the previous diagonal
        load_x(s + 1, xn);                                    // prefetch; consumed next step
        const float* prev = lds + ((s + 1) & 1) * ROWS * RS;
        float* cur = lds + (s & 1) * ROWS * RS;
        f32x4 acc[5];
#pragma unroll
        for (int g = 0; g < 5; ++g) acc[g] = f32x4{bz[g], bz[g], bz[g], bz[g]};
        if (mt * 16 < L) {  // uniform over the wave
            const int a = lo + ja, b = s - a;
            const int rl = (ja < L && b > 0) ? ja + dl : ZR;      // left predecessor (a, b-1)
            const int ru = (ja < L && a > 0) ? ja + dl - 1 : ZR;  // upper predecessor (a-1, b)
#pragma unroll
            for (int ks = 0; ks < kMaxKX; ++ks)
                if (ks < KX)
#pragma unroll
                    for (int g = 0; g < 5; ++g)
                        acc[g] = __builtin_amdgcn_mfma_f32_16x16x4f32(xv[ks], Bx[g][ks], acc[g], 0, 0, 0);
#pragma unroll
            for (int ks = 0; ks < KP; ++ks) {
                const int n = 4 * ks + krow;
                const int row = n < H ? rl : (n < 2 * H ? ru : ZR);
                const int cn = n < H ? n : (n < 2 * H ? n - H : 0);
                const float ah = prev[row * RS + cn], as = prev[row * RS + H + cn];
#pragma unroll
                for (int g = 0; g < 5; ++g) acc[g] = __builtin_amdgcn_mfma_f32_16x16x4f32(ah, Bh[g][ks], acc[g], 0, 0, 0);
#pragma unroll
                for (int m = 0; m < 3; ++m)
                    acc[1 + m] = __builtin_amdgcn_mfma_f32_16x16x4f32(as, Bs[m][ks], acc[1 + m], 0, 0, 0);
            }
        }
        const int kc = kok ? kk : 0;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int jo = mt * 16 + 4 * krow + r;
            const int a = lo + jo, b = s - a;
            const bool ok = (jo < L) & kok;
            const float sl = prev[((jo < L && b > 0) ? jo + dl : ZR) * RS + H + kc];
            const float su = prev[((jo < L && a > 0) ? jo + dl - 1 : ZR) * RS + H + kc];
            const float f = sigm(acc[0][r]), lam = sigm(acc[1][r]), o1 = sigm(acc[2][r]), o2 = sigm(acc[3][r]);
            const float gg = ftanh(acc[4][r]);
            const float sbar = __builtin_fmaf(lam, sl - su, su);
            const float sv = __builtin_fmaf(f, sbar - gg, gg);
            const float hv = __builtin_fmaf(o1, ftanh(sv), o2 * sv);
            if (ok) {
                cur[jo * RS + kk] = hv;
                cur[jo * RS + H + kk] = sv;
            }
            const int el = (st + jo) * H + kc;
            const int ho = ok ? ((F.y(a) * D.Wc + F.x(b)) * H + kk) * 4 : kOOBl;
            bst(hv, rH, ho);
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, f32x4{f, lam, o1, o2}), rS4,
                                                   ok ? el * 16 : kOOBl, 0, 0);
            __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, f32x2{gg, sv}), rS2, ok ? el * 8 : kOOBl,
                                                  0, 0);
        }
        __syncthreads();
    };
    int s = 0;
    for (; s + 1 < S; s += 2) {
        step(s, xa, xb);
        step(s + 1, xb, xa);
    }
    if (s < S) step(s, xa, xb);
}

// Reverse wavefront. The upstream gradient is dy_flat (the direction sum's, the same for every direction) or
// dh_dirs [4][Hc][Wc][H]. For cell (a, b) with successors R = (a, b+1), D = (a+1, b) on the later diagonal:
//     dh    = dy + da(R).Ul^T + da(D).Uu^T
//     ds_in = ds_l(R) + ds_u(D) + da3(R).Vl^T + da3(D).Vu^T      (da3: the lam, o1, o2 columns)
// where ds_l(R) = dsbar(R) lam(R) is what R sends to its left predecessor, ds_u(D) = dsbar(D) (1 - lam(D)).
template <int H>
__global__ __launch_bounds__(LeakyShape<H>::MAXT) void k_bwd_leaky(Dev D, int NT, const float* __restrict__ Ul,
                                                    const float* __restrict__ Uu, const float* __restrict__ Vl,
                                                    const float* __restrict__ Vu, const float* __restrict__ stash,
                                                    const float* __restrict__ dy_flat,
                                                    const float* __restrict__ dh_dirs, float* __restrict__ dA) {
    using Sh = LeakyShape<H>;
    constexpr int NB = Sh::NB, RG = Sh::RG, RD = Sh::RD, G = 5 * H, G3 = 3 * H;
    constexpr int KU = (2 * G + 3) / 4;   // k-steps over [da(R) | da(D)]
    constexpr int KV = (2 * G3 + 3) / 4;  // k-steps over [da3(R) | da3(D)]
    const int u = D.units[blockIdx.x];
    const int e = u >> 2, d = u & 3;
    const Flip F{D.rect[4 * e], D.rect[4 * e + 1], D.rect[4 * e + 2], D.rect[4 * e + 3], (d & 2) != 0, (d & 1) != 0};
    const int h = F.h, w = F.w;
    const int ry0 = D.real[4 * e], rx0 = D.real[4 * e + 1], rh = D.real[4 * e + 2], rw = D.real[4 * e + 3];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int mt = wave / NB, kb = wave % NB;
    const int col = lane & 15, krow = lane >> 4;
    const int kk = kb * 16 + col;
    const bool kok = kk < H;
    const int kc = kok ? kk : 0;

    // B fragments: [Ul^T; Uu^T] and [Vl^T; Vu^T], row 4 ks + krow, column kk
    float BU[KU], BV[KV];
#pragma unroll
    for (int ks = 0; ks < KU; ++ks) {
        const int n = 4 * ks + krow;
        float v = 0.f;
        if (kok && n < G) v = Ul[((int64_t)d * H + kk) * G + n];
        else if (kok && n < 2 * G) v = Uu[((int64_t)d * H + kk) * G + n - G];
        BU[ks] = v;
    }
#pragma unroll
    for (int ks = 0; ks < KV; ++ks) {
        const int n = 4 * ks + krow;
        float v = 0.f;
        if (kok && n < G3) v = Vl[((int64_t)d * H + kk) * G3 + n];
        else if (kok && n < 2 * G3) v = Vu[((int64_t)d * H + kk) * G3 + n - G3];
        BV[ks] = v;
    }

    extern __shared__ __align__(16) float lds[];
    const int ZR = 16 * NT, ROWS = ZR + 1;
    float* dab = lds;                     // [2][ROWS][RG] gate gradients of a diagonal
    float* dsl = dab + 2 * ROWS * RG;     // [2][ROWS][RD] ds sent to the left predecessor
    float* dsu = dsl + 2 * ROWS * RD;     // [2][ROWS][RD] ds sent to the upper predecessor
    for (int i = threadIdx.x; i < 2 * ROWS * (RG + 2 * RD); i += blockDim.x) lds[i] = 0.f;

    const int64_t base = (int64_t)d * D.T + D.cell_off[e];
    const int64_t cells = (int64_t)h * w;
    const __amdgpu_buffer_rsrc_t rS4 = rsrc(stash + base * 4 * H, cells * 16 * H);
    const __amdgpu_buffer_rsrc_t rS2 = rsrc(stash + z1_offset(D.T, H) + base * 2 * H, cells * 8 * H);
    const __amdgpu_buffer_rsrc_t rA4 = rsrc(dA + base * 4 * H, cells * 16 * H);
    const __amdgpu_buffer_rsrc_t rA1 = rsrc(dA + z1_offset(D.T, H) + base * H, cells * 4 * H);
    const bool per_dir = dh_dirs != nullptr;
    const __amdgpu_buffer_rsrc_t rU =
        per_dir ? rsrc(dh_dirs + (int64_t)d * D.Hc * D.Wc * H, (int64_t)D.Hc * D.Wc * H * 4)
                : rsrc(dy_flat + D.flat_off[e] * H, (int64_t)rh * rw * H * 4);
    const int S = h + w - 1;

    // per output row r: f, lam, o1, o2, g, s, s_left, s_up, upstream dh
    auto load_v = [&](int s, float (&v)[9][4]) {
        const bool in = s >= 0;
        const int L = in ? dg_len(h, w, s) : 0, lo = in ? dg_lo(h, w, s) : 0;
        const int st = in ? (int)dg_start(h, w, s) : 0;
        const int lop = s > 0 ? dg_lo(h, w, s - 1) : 0;
        const int stp = s > 0 ? (int)dg_start(h, w, s - 1) : 0;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int jo = mt * 16 + 4 * krow + r;
            const bool ok = (jo < L) & kok;
            const int a = lo + jo, b = s - a;
            const int ei = (st + jo) * H + kc;
            const int so4 = ok ? ei * 16 : kOOBl, so2 = ok ? ei * 8 : kOOBl;
            const f32x4 g4 = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rS4, so4, 0, 0));
            const f32x2 g2 = __builtin_bit_cast(f32x2, __builtin_amdgcn_raw_buffer_load_b64(rS2, so2, 0, 0));
            v[0][r] = g4[0]; v[1][r] = g4[1]; v[2][r] = g4[2]; v[3][r] = g4[3];
            v[4][r] = g2[0]; v[5][r] = g2[1];
            v[6][r] = bld(rS2, (ok && b > 0) ? (((stp + a - lop) * H + kc) * 2 + 1) * 4 : kOOBl);
            v[7][r] = bld(rS2, (ok && a > 0) ? (((stp + a - 1 - lop) * H + kc) * 2 + 1) * 4 : kOOBl);
            const int y = F.y(a), x = F.x(b);
            const int ly = y - ry0, lx = x - rx0;
            int uo = kOOBl;
            if (ok && per_dir) uo = ((y * D.Wc + x) * H + kk) * 4;
            if (ok && !per_dir && ly >= 0 && lx >= 0 && ly < rh && lx < rw) uo = ((ly * rw + lx) * H + kk) * 4;
            v[8][r] = bld(rU, uo);
        }
    };

    auto step = [&](int s, const float (&vc)[9][4], float (&vn)[9][4]) {
        const int L = dg_len(h, w, s), lo = dg_lo(h, w, s);
        const int st = (int)dg_start(h, w, s);
        const int lon = s + 1 < S ? dg_lo(h, w, s + 1) : 0;
        load_v(s - 1, vn);  // prefetch; consumed next step
        const float* dar = dab + ((s + 1) & 1) * ROWS * RG;
        const float* dslr = dsl + ((s + 1) & 1) * ROWS * RD;
        const float* dsur = dsu + ((s + 1) & 1) * ROWS * RD;
        float* daw = dab + (s & 1) * ROWS * RG;
        float* dslw = dsl + (s & 1) * ROWS * RD;
        float* dsuw = dsu + (s & 1) * ROWS * RD;
        f32x4 ah = f32x4{vc[8][0], vc[8][1], vc[8][2], vc[8][3]};
        f32x4 as = f32x4{0.f, 0.f, 0.f, 0.f};
        if (mt * 16 < L) {  // uniform over the wave
            const int j = mt * 16 + col;
            const int a = lo + j, b = s - a;
            const int jr = (j < L && b + 1 < w) ? a - lon : ZR;      // right successor (a, b+1)
            const int jd = (j < L && a + 1 < h) ? a + 1 - lon : ZR;  // lower successor (a+1, b)
            f32x4 ah2 = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KU; ++ks) {
                const int n = 4 * ks + krow;
                const float av = dar[n < G ? jr * RG + n : (n < 2 * G ? jd * RG + n - G : ZR * RG)];
                if (ks & 1) ah2 = __builtin_amdgcn_mfma_f32_16x16x4f32(av, BU[ks], ah2, 0, 0, 0);
                else ah = __builtin_amdgcn_mfma_f32_16x16x4f32(av, BU[ks], ah, 0, 0, 0);
            }
            ah += ah2;
#pragma unroll
            for (int ks = 0; ks < KV; ++ks) {
                const int n = 4 * ks + krow;
                const float av = dar[n < G3 ? jr * RG + H + n : (n < 2 * G3 ? jd * RG + H + n - G3 : ZR * RG)];
                as = __builtin_amdgcn_mfma_f32_16x16x4f32(av, BV[ks], as, 0, 0, 0);
            }
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int jo = mt * 16 + 4 * krow + r;
            const int a = lo + jo, b = s - a;
            const bool ok = (jo < L) & kok;
            const float dsin = as[r] + dslr[((jo < L && b + 1 < w) ? a - lon : ZR) * RD + kc] +
                               dsur[((jo < L && a + 1 < h) ? a + 1 - lon : ZR) * RD + kc];
            const float dh = ah[r];
            const float f = vc[0][r], lam = vc[1][r], o1 = vc[2][r], o2 = vc[3][r];
            const float gg = vc[4][r], sv = vc[5][r], sl = vc[6][r], su = vc[7][r];
            const float ts = ftanh(sv);
            const float ds = __builtin_fmaf(dh, __builtin_fmaf(o1, 1.f - ts * ts, o2), dsin);
            const float sbar = __builtin_fmaf(lam, sl - su, su);
            const float dsbar = ds * f;
            const float d0 = ds * (sbar - gg) * f * (1.f - f);
            const float d1 = dsbar * (sl - su) * lam * (1.f - lam);
            const float d2 = dh * ts * o1 * (1.f - o1);
            const float d3 = dh * sv * o2 * (1.f - o2);
            const float d4 = ds * (1.f - f) * (1.f - gg * gg);
            if (ok) {
                float* dw = daw + jo * RG + kk;
                dw[0] = d0; dw[H] = d1; dw[2 * H] = d2; dw[3 * H] = d3; dw[4 * H] = d4;
                dslw[jo * RD + kk] = dsbar * lam;
                dsuw[jo * RD + kk] = dsbar - dsbar * lam;
            }
            const int ea = (st + jo) * H + kc;
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, f32x4{d0, d1, d2, d3}), rA4,
                                                   ok ? ea * 16 : kOOBl, 0, 0);
            bst(d4, rA1, ok ? ea * 4 : kOOBl);
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

// Weight gradients of the memory-state projections, one workgroup per weight-gradient range (the layout's
// split of the computed cells into segments), one wave per direction:
//     dVl[d] = sum over cells of s_l (x) da3,   dVu[d] = sum over cells of s_u (x) da3
// as [s_l | s_u]^T (2H x cells) times da3 (cells x 3H) on v_mfma_f32_16x16x4_f32, 16 cells per tile. Each
// workgroup writes its partial [4][2H][3H]; k_dv_reduce adds the partials in workgroup order.
template <int H>
__global__ __launch_bounds__(256) void k_dv_leaky(Dev D, const float* __restrict__ stash,
                                                  const float* __restrict__ dA, float* __restrict__ part) {
    constexpr int MB = (2 * H + 15) / 16, NB3 = (3 * H + 15) / 16, G3 = 3 * H;
    const int grp = blockIdx.x;
    const int d = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int col = lane & 15, krow = lane >> 4;
    f32x4 acc[MB][NB3];
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int j = 0; j < NB3; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    const float* S2 = stash + z1_offset(D.T, H) + (int64_t)d * D.T * 2 * H;
    const float* A4 = dA + (int64_t)d * D.T * 4 * H;
    for (int sg = D.groups[grp]; sg < D.groups[grp + 1]; ++sg) {
        const int e = D.segs[3 * sg], c0 = D.segs[3 * sg + 1], c1 = D.segs[3 * sg + 2];
        const int h = D.rect[4 * e + 2], w = D.rect[4 * e + 3];
        const int64_t cb = D.cell_off[e];
        for (int t0 = c0; t0 < c1; t0 += 16) {
            // lane's cells: k-step q holds cell t0 + 4 q + krow (region-local, row-major)
            float av[4][MB], bv[4][NB3];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int c = t0 + 4 * q + krow;
                const bool in = c < c1;
                const int ly = in ? c / w : 0, lx = in ? c - (c / w) * w : 0;
                const int a = (d & 2) ? h - 1 - ly : ly, b = (d & 1) ? w - 1 - lx : lx;
                const int s = a + b;
                const int64_t ic = cb + dg_start(h, w, s) + a - dg_lo(h, w, s);
                const int64_t ip = s > 0 ? cb + dg_start(h, w, s - 1) - dg_lo(h, w, s - 1) : 0;  // + row
#pragma unroll
                for (int mb = 0; mb < MB; ++mb) {
                    const int m = 16 * mb + col;  // row of [s_l | s_u]
                    float v = 0.f;
                    if (in && m < H && b > 0) v = S2[((ip + a) * H + m) * 2 + 1];
                    else if (in && m >= H && m < 2 * H && a > 0) v = S2[((ip + a - 1) * H + m - H) * 2 + 1];
                    av[q][mb] = v;
                }
#pragma unroll
                for (int nb = 0; nb < NB3; ++nb) {
                    const int n = 16 * nb + col;  // column of da3: gate 1 + n / H, unit n % H
                    bv[q][nb] = (in && n < G3) ? A4[(ic * H + n % H) * 4 + 1 + n / H] : 0.f;
                }
            }
#pragma unroll
            for (int q = 0; q < 4; ++q)
#pragma unroll
                for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                    for (int nb = 0; nb < NB3; ++nb)
                        acc[mb][nb] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[q][mb], bv[q][nb], acc[mb][nb], 0, 0, 0);
        }
    }
    float* out = part + ((int64_t)grp * 4 + d) * (2 * H) * G3;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < NB3; ++nb)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int m = 16 * mb + 4 * krow + r, n = 16 * nb + col;
                if (m < 2 * H && n < G3) out[(int64_t)m * G3 + n] = acc[mb][nb][r];
            }
}

// dVl, dVu: the partials of k_dv_leaky added in workgroup order, one thread per entry
__global__ __launch_bounds__(256) void k_dv_reduce(const float* __restrict__ part, int ngroups, int H,
                                                   float* __restrict__ dVl, float* __restrict__ dVu) {
    const int E = 2 * H * 3 * H;
    const int id = blockIdx.x * blockDim.x + threadIdx.x;
    if (id >= 4 * E) return;
    float s = 0.f;
    for (int g = 0; g < ngroups; ++g) s += part[(int64_t)g * 4 * E + id];
    const int d = id / E, rem = id - d * E, m = rem / (3 * H), n = rem - m * 3 * H;
    if (m < H) dVl[((int64_t)d * H + m) * 3 * H + n] = s;
    else dVu[((int64_t)d * H + m - H) * 3 * H + n] = s;
}

typedef void (*FwdLeakyK)(Dev, const void*, int, int, const float*, const float*, const float*, const float*,
                          const float*, const float*, float*, float*);
typedef void (*BwdLeakyK)(Dev, int, const float*, const float*, const float*, const float*, const float*,
                          const float*, const float*, float*);
typedef void (*DvLeakyK)(Dev, const float*, const float*, float*);

struct LeakyEntry {
    int H;
    FwdLeakyK fwd[2];  // f32, bf16 input
    BwdLeakyK bwd;
    DvLeakyK dv;
    int NB, MAXT;
};
#define MDL_LK(h)                                                                                          \
    {h, {k_fwd_leaky<h, false>, k_fwd_leaky<h, true>}, k_bwd_leaky<h>, k_dv_leaky<h>, LeakyShape<h>::NB, \
     LeakyShape<h>::MAXT}
const LeakyEntry kLeaky[] = {MDL_LK(4), MDL_LK(8), MDL_LK(16), MDL_LK(32)};
#undef MDL_LK

const LeakyEntry* leaky_entry(int H) {
    for (const auto& m : kLeaky)
        if (m.H == H) return &m;
    return nullptr;
}

int leaky_tiles(int Lmax) { return (Lmax + 15) / 16; }

}  // namespace

bool leaky_supported(int H, int C, int Lmax) {
    const LeakyEntry* m = leaky_entry(H);
    return m && C >= 1 && C <= 4 * kMaxKX && 64 * leaky_tiles(Lmax) * m->NB <= m->MAXT;
}

size_t leaky_fwd_lds(int H, int Lmax) {
    if (leaky16_used(H, Lmax)) return leaky16_fwd_lds(H, Lmax);
    return sizeof(float) * 2 * (size_t)(16 * leaky_tiles(Lmax) + 1) * (2 * H + 4);
}

size_t leaky_bwd_lds(int H, int Lmax) {
    if (leaky16_used(H, Lmax)) return leaky16_bwd_lds(H, Lmax);
    return sizeof(float) * 2 * (size_t)(16 * leaky_tiles(Lmax) + 1) * ((5 * H + 4) + 2 * (H + 4));
}

hipError_t launch_fwd_leaky(const Dev& D, const void* x_canvas, int dtype, int C, int H, const float* Wx,
                            const float* b, const float* Ul, const float* Uu, const float* Vl, const float* Vu,
                            float* stash, float* h_dirs, hipStream_t st) {
    if (leaky16_used(H, D.max_diag))
        return launch_fwd_leaky16(D, x_canvas, dtype, C, H, Wx, b, Ul, Uu, Vl, Vu, stash, h_dirs, st);
    const LeakyEntry* m = leaky_entry(H);
    if (!m) return hipErrorInvalidValue;
    const int NT = leaky_tiles(D.max_diag);
    launch(m->fwd[dtype != 0 ? 1 : 0], dim3(4 * D.n), dim3(64 * NT * m->NB), leaky_fwd_lds(H, D.max_diag), st, D,
           x_canvas, C, NT, Wx, b, Ul, Uu, Vl, Vu, stash, h_dirs);
    return hipGetLastError();
}

hipError_t launch_bwd_leaky(const Dev& D, int H, const float* Ul, const float* Uu, const float* Vl, const float* Vu,
                            const float* stash, const float* dy_flat, const float* dh_dirs, float* dA,
                            hipStream_t st) {
    if (leaky16_used(H, D.max_diag))
        return launch_bwd_leaky16(D, H, Ul, Uu, Vl, Vu, stash, dy_flat, dh_dirs, dA, nullptr, st);
    const LeakyEntry* m = leaky_entry(H);
    if (!m) return hipErrorInvalidValue;
    const int NT = leaky_tiles(D.max_diag);
    launch(m->bwd, dim3(4 * D.n), dim3(64 * NT * m->NB), leaky_bwd_lds(H, D.max_diag), st, D, NT, Ul, Uu, Vl, Vu,
           stash, dy_flat, dh_dirs, dA);
    return hipGetLastError();
}

hipError_t launch_dv_leaky(const Dev& D, int H, const float* stash, const float* dA, float* part, float* dVl,
                           float* dVu, hipStream_t st) {
    const LeakyEntry* m = leaky_entry(H);
    if (!m) return hipErrorInvalidValue;
    launch(m->dv, dim3(D.ngroups), dim3(256), 0, st, D, stash, dA, part);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int n = 4 * 2 * H * 3 * H;
    launch(k_dv_reduce, dim3((n + 255) / 256), dim3(256), 0, st, part, D.ngroups, H, dVl, dVu);
    return hipGetLastError();
}

}  // namespace mdl
