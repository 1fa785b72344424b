// k_leaky16.hip — the Leaky-LP cell's wavefronts ("No Padding Please" §III, Figure 4(b); §IX-A) with the
// recurrent products on the 16-bit matrix instructions, for hidden sizes 16 and 32.
//
// Same cell, schedule, work split and stash layout as k_leaky.hip (one workgroup per (example, direction)
// unit walks its local anti-diagonals; wave (tile mt, block kb) owns 16 cells of the diagonal and 16
// hidden units); only the products change. There each 4-wide K step is one v_mfma_f32_16x16x4_f32; here
// each 32-wide K block takes four (forward) or six (reverse) 16-bit instructions of eight times the
// multiply-adds per cycle, with operands split into pieces so that the products stay those of fp32:
//
// - Forward, a[g] += [h_l, h_u].[Ul; Uu] (five gates) and [s_l, s_u].[Vl; Vu] (lam, o1, o2), on
//   v_mfma_f32_16x16x32_f16. The states are bounded (|s| < 1, |h| < 2: both are convex combinations of
//   values in (-1, 1), h of tanh s and s), so h and s are scaled by 2^13 and split into f16 pairs,
//   hi + lo (about 22 bits). Each gate column of the weights (U and V of a gate share its accumulator)
//   is scaled by its own power of two and split into three f16 pieces hi + lo + r, exact to about 2^-33.
//   The four terms h_hi.r + h_lo.U_hi + h_hi.U_lo + h_hi.U_hi are kept, smallest first, and the
//   accumulator is scaled back exactly (with the base-2 fold of the sigmoid gates) before x.Wx + b is
//   added. The pieces of h and s are written to LDS once, by the lane that computes them.
// - Reverse, dh += [da(R), da(D)].[Ul^T; Uu^T] and ds += [da3(R), da3(D)].[Vl^T; Vu^T], on
//   v_mfma_f32_16x16x32_bf16. The gate gradients are unbounded, and bf16 keeps fp32's exponent range,
//   so nothing is scaled: every fp32 operand is split exactly into three bf16 pieces v1 + v2 + v3 (each
//   the leading 8 significant bits of what the ones before leave) and the six terms v_i w_j with
//   i + j <= 4 are kept, smallest first (each dropped term is below 2^-23 of v w). The gate gradients' pieces are written to
//   LDS by the lane that computes them.
#include "kernels.h"
#include "leaky16.h"
#include "devmath.h"

namespace mdl {

namespace {

constexpr int kOOB6 = 0x40000000;  // byte offset past every per-unit range used here (1 GiB)
constexpr int kMaxKX6 = 4;         // input channels up to 16
constexpr float kL2E6 = 1.44269504088896341f;
constexpr float kHS6 = 8192.f;      // 2^13: h in (-2, 2) and s in (-1, 1) -> f16 range
// sigmoid gates (f, lam, o1, o2) take their argument as a base-2 exponent: sigmoid(a) = 1 / (1 + 2^(-a log2 e))
__host__ __device__ constexpr float lk_fold(int g) { return g < 4 ? -kL2E6 : 1.0f; }
__device__ inline float lk_sig(float t) { return frcp(1.0f + __builtin_amdgcn_exp2f(t)); }

typedef __bf16 bf16x8_l __attribute__((ext_vector_type(8)));

template <int H>
struct LK16 {
    static_assert(H % 16 == 0, "hidden size a multiple of 16");
    static constexpr int NB = H / 16;               // 16-wide blocks of hidden units
    static constexpr int G = 5 * H, G3 = 3 * H;
    static constexpr int KB = (2 * H + 31) / 32;    // forward K blocks over [left | up]
    static constexpr int RSH = 4 * H + 8;           // forward LDS row (halves): h hi, h lo, s hi, s lo
    static constexpr int CS = H + 4;                // forward LDS row (floats): s
    static constexpr int KU = 2 * G / 32;           // reverse K blocks over [da(R) | da(D)]
    static constexpr int KV = (2 * G3 + 31) / 32;   // ... over [da3(R) | da3(D)]
    static constexpr int RGB = 3 * G + 8;           // reverse LDS row (halves): the three bf16 pieces of da
    static constexpr int RD = H + 4;                // reverse LDS row (floats): ds sent to a predecessor
    static constexpr int MAXT = NB >= 2 ? 256 : 512;
    static_assert(2 * G % 32 == 0 && 2 * G3 % 32 == 0, "whole K blocks");
};

// the exact three-piece bf16 split of eight fp32 values (pairs packed low: even, high: odd)
__device__ inline void split3b(const float (&v)[8], u32x4 (&p)[3]) {
    uint32_t u[3][8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const uint32_t b0 = __float_as_uint(v[i]);
        const float e1 = v[i] - __uint_as_float(b0 & 0xFFFF0000u);
        const uint32_t b1 = __float_as_uint(e1);
        const float e2 = e1 - __uint_as_float(b1 & 0xFFFF0000u);
        u[0][i] = b0;
        u[1][i] = b1;
        u[2][i] = __float_as_uint(e2);
    }
#pragma unroll
    for (int k = 0; k < 3; ++k)
#pragma unroll
        for (int i = 0; i < 4; ++i) p[k][i] = __builtin_amdgcn_perm(u[k][2 * i + 1], u[k][2 * i], 0x07060302u);
}

// the same split of one value, as three bf16 bit patterns
__device__ inline void split3b1(float v, uint16_t& p0, uint16_t& p1, uint16_t& p2) {
    const uint32_t b0 = __float_as_uint(v);
    const float e1 = v - __uint_as_float(b0 & 0xFFFF0000u);
    const uint32_t b1 = __float_as_uint(e1);
    const float e2 = e1 - __uint_as_float(b1 & 0xFFFF0000u);
    p0 = (uint16_t)(b0 >> 16);
    p1 = (uint16_t)(b1 >> 16);
    p2 = (uint16_t)(__float_as_uint(e2) >> 16);
}

__device__ inline f32x4 mfma_bf(const u32x4& a, const u32x4& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_l, a), __builtin_bit_cast(bf16x8_l, b),
                                                   c, 0, 0, 0);
}

// Forward. KX: K steps of 4 input channels; XBF: canvas pixels stored as bf16.
template <int H, int KX, bool XBF>
__global__ __launch_bounds__(LK16<H>::MAXT) void k_fwd_leaky16(Dev D, const void* __restrict__ xc, int C, int NT,
                                                             const float* __restrict__ Wx,
                                                             const float* __restrict__ bias,
                                                             const float* __restrict__ Ul,
                                                             const float* __restrict__ Uu,
                                                             const float* __restrict__ Vl,
                                                             const float* __restrict__ Vu, float* __restrict__ stash,
                                                             float* __restrict__ hdirs) {
    using Sh = LK16<H>;
    constexpr int NB = Sh::NB, KB = Sh::KB, RSH = Sh::RSH, CS = Sh::CS, G = Sh::G, G3 = Sh::G3;
    const int u = D.units[blockIdx.x];
    const int e = u >> 2, d = u & 3;
    const Flip F{D.rect[4 * e], D.rect[4 * e + 1], D.rect[4 * e + 2], D.rect[4 * e + 3], (d & 2) != 0, (d & 1) != 0};
    const int h = F.h, w = F.w;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int mt = wave / NB, kb = wave % NB;
    const int col = lane & 15, q = lane >> 4;
    const int kk = kb * 16 + col;  // this lane's hidden unit (output column); every lane has one

    // B pieces: lane holds K rows 32 t + 8 q .. + 7 of column kk of gate g: [Ul; Uu] (Ul row k at K index k,
    // Uu row k at H + k) and, for lam, o1, o2, [Vl; Vu] likewise; scaled per gate column by 2^E[g].
    auto wu = [&](int g, int k) {
        return k < H ? Ul[((int64_t)d * H + k) * G + g * H + kk] : Uu[((int64_t)d * H + k - H) * G + g * H + kk];
    };
    auto wv = [&](int m, int k) {
        return k < H ? Vl[((int64_t)d * H + k) * G3 + m * H + kk] : Vu[((int64_t)d * H + k - H) * G3 + m * H + kk];
    };
    int E[5];
    float us[5];  // 2^-(E + 13) times the gate's fold: undoes both scalings
#pragma unroll
    for (int g = 0; g < 5; ++g) {
        float m = 0.f;
#pragma unroll
        for (int t = 0; t < KB; ++t)
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int k = 32 * t + 8 * q + i;
                if (k < 2 * H) {
                    m = fmaxf(m, fabsf(wu(g, k)));
                    if (g >= 1 && g <= 3) m = fmaxf(m, fabsf(wv(g - 1, k)));
                }
            }
        m = fmaxf(m, __shfl_xor(m, 16));
        m = fmaxf(m, __shfl_xor(m, 32));
        int Eg = 0;
        if (m > 0.f) {
            Eg = 14 - ((int)((__float_as_uint(m) >> 23) & 255) - 127);
            Eg = Eg < -100 ? -100 : (Eg > 100 ? 100 : Eg);
        }
        E[g] = Eg;
        us[g] = ldexpf(1.0f, -(Eg + 13)) * lk_fold(g);
    }
    auto split_col = [&](float x, int Eg, _Float16& hi, _Float16& lo, _Float16& r) {
        const float vs = ldexpf(x, Eg);
        split16(vs, hi, lo);
        // vs - hi and then - lo are exact in fp32 (each operand holds the leading bits of the other)
        r = (_Float16)((vs - (float)hi) - (float)lo);
    };
    f16x8 Uh[5][KB], Uo[5][KB], Ur[5][KB], Vh[3][KB], Vo[3][KB], Vr[3][KB];
#pragma unroll
    for (int g = 0; g < 5; ++g)
#pragma unroll
        for (int t = 0; t < KB; ++t)
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int k = 32 * t + 8 * q + i;
                _Float16 a0, a1, a2;
                split_col(k < 2 * H ? wu(g, k) : 0.f, E[g], a0, a1, a2);
                Uh[g][t][i] = a0;
                Uo[g][t][i] = a1;
                Ur[g][t][i] = a2;
            }
#pragma unroll
    for (int m = 0; m < 3; ++m)
#pragma unroll
        for (int t = 0; t < KB; ++t)
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int k = 32 * t + 8 * q + i;
                _Float16 a0, a1, a2;
                split_col(k < 2 * H ? wv(m, k) : 0.f, E[1 + m], a0, a1, a2);
                Vh[m][t][i] = a0;
                Vo[m][t][i] = a1;
                Vr[m][t][i] = a2;
            }
    // input projection on the fp32 matrix instruction, the fold applied to the weights and the bias
    float Bx[5][KX], bz[5];
#pragma unroll
    for (int g = 0; g < 5; ++g) {
        bz[g] = bias[(int64_t)d * G + g * H + kk] * lk_fold(g);
#pragma unroll
        for (int ks = 0; ks < KX; ++ks) {
            const int c = 4 * ks + q;
            Bx[g][ks] = c < C ? Wx[((int64_t)d * C + c) * G + g * H + kk] * lk_fold(g) : 0.f;
        }
    }

    // LDS, two buffers (previous / current diagonal): rows of the f16 pieces of 2^13 h and 2^13 s, then rows
    // of s in fp32 (for the lambda gate's convex combination); row j is diagonal position j, row ZR zeros,
    // row XR takes the writes of lanes without a cell. The step has no branch: the compiler would wait for
    // every store in flight where control flow merges (loads and stores retire in order here).
    extern __shared__ __align__(16) unsigned char smem[];
    const int ZR = 16 * NT, XR = ZR + 1, ROWS = ZR + 2;
    const int HBUF = ROWS * RSH * 2, SBUF = ROWS * CS * 4;
    {
        uint32_t* z32 = reinterpret_cast<uint32_t*>(smem);
        for (int i = threadIdx.x; i < (HBUF + SBUF) / 2; i += blockDim.x) z32[i] = 0u;
    }

    const int64_t base = (int64_t)d * D.T + D.cell_off[e];
    const int64_t cells = (int64_t)h * w;
    const int XB = XBF ? 2 : 4;
    const __amdgpu_buffer_rsrc_t rX = rsrc(xc, (int64_t)D.Hc * D.Wc * C * XB);
    const __amdgpu_buffer_rsrc_t rS4 = rsrc(stash + base * 4 * H, cells * 16 * H);
    const __amdgpu_buffer_rsrc_t rS2 = rsrc(stash + z1_offset(D.T, H) + base * 2 * H, cells * 8 * H);
    const __amdgpu_buffer_rsrc_t rH = rsrc(hdirs + (int64_t)d * D.Hc * D.Wc * H, (int64_t)D.Hc * D.Wc * H * 4);
    const int S = h + w - 1;
    const int ja = mt * 16 + col;  // this lane's A row: its cell on the diagonal

    auto load_x = [&](int s1, float (&xv)[KX]) {
        const bool in = s1 < S;
        const int L1 = in ? dg_len(h, w, s1) : 0, lo1 = in ? dg_lo(h, w, s1) : 0;
        const int a = lo1 + ja, b = s1 - a;
        const bool va = ja < L1;
        const int px = va ? F.y(a) * D.Wc + F.x(b) : 0;
#pragma unroll
        for (int ks = 0; ks < KX; ++ks) {
            const int c = 4 * ks + q;
            const int off = (va && c < C) ? (px * C + c) * XB : kOOB6;
            if constexpr (XBF)
                xv[ks] = __uint_as_float((uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rX, off, 0, 0) << 16);
            else
                xv[ks] = bld(rX, off);
        }
    };
    float xa[KX], xb[KX];
    load_x(0, xa);
    __syncthreads();

    auto step = [&](int s, const float (&xv)[KX], float (&xn)[KX]) {
        const int L = dg_len(h, w, s), lo = dg_lo(h, w, s);
        const int st = (int)dg_start(h, w, s);
        const int dl = s > 0 ? lo - dg_lo(h, w, s - 1) : 0;  // position shift to the previous diagonal
        load_x(s + 1, xn);                                    // prefetch; consumed next step
        const unsigned char* hp = smem + ((s + 1) & 1) * HBUF;
        const float* sp = reinterpret_cast<const float*>(smem + 2 * HBUF + ((s + 1) & 1) * SBUF);
        unsigned char* hc = smem + (s & 1) * HBUF;
        float* sc = reinterpret_cast<float*>(smem + 2 * HBUF + (s & 1) * SBUF);
        f32x4 acc[5], accx[5];
#pragma unroll
        for (int g = 0; g < 5; ++g) {
            acc[g] = f32x4{0.f, 0.f, 0.f, 0.f};
            accx[g] = f32x4{bz[g], bz[g], bz[g], bz[g]};
        }
        {
            const int a = lo + ja, b = s - a;
            const int rl = (ja < L && b > 0) ? ja + dl : ZR;      // left predecessor (a, b-1)
            const int ru = (ja < L && a > 0) ? ja + dl - 1 : ZR;  // upper predecessor (a-1, b)
#pragma unroll
            for (int ks = 0; ks < KX; ++ks)
#pragma unroll
                for (int g = 0; g < 5; ++g)
                    accx[g] = __builtin_amdgcn_mfma_f32_16x16x4f32(xv[ks], Bx[g][ks], accx[g], 0, 0, 0);
#pragma unroll
            for (int t = 0; t < KB; ++t) {
                const int k0 = 32 * t + 8 * q;
                const int row = k0 < H ? rl : (k0 < 2 * H ? ru : ZR);
                const int off = k0 < H ? k0 : (k0 < 2 * H ? k0 - H : 0);
                const unsigned char* p = hp + row * (RSH * 2) + off * 2;
                const f16x8 Ah = *reinterpret_cast<const f16x8*>(__builtin_assume_aligned(p, 16));
                const f16x8 Al = *reinterpret_cast<const f16x8*>(__builtin_assume_aligned(p + 2 * H, 16));
                const f16x8 Sa = *reinterpret_cast<const f16x8*>(__builtin_assume_aligned(p + 4 * H, 16));
                const f16x8 Sl = *reinterpret_cast<const f16x8*>(__builtin_assume_aligned(p + 6 * H, 16));
#pragma unroll
                for (int g = 0; g < 5; ++g) {
                    acc[g] = __builtin_amdgcn_mfma_f32_16x16x32_f16(Ah, Ur[g][t], acc[g], 0, 0, 0);
                    acc[g] = __builtin_amdgcn_mfma_f32_16x16x32_f16(Al, Uh[g][t], acc[g], 0, 0, 0);
                    acc[g] = __builtin_amdgcn_mfma_f32_16x16x32_f16(Ah, Uo[g][t], acc[g], 0, 0, 0);
                    acc[g] = __builtin_amdgcn_mfma_f32_16x16x32_f16(Ah, Uh[g][t], acc[g], 0, 0, 0);
                }
#pragma unroll
                for (int m = 0; m < 3; ++m) {
                    acc[1 + m] = __builtin_amdgcn_mfma_f32_16x16x32_f16(Sa, Vr[m][t], acc[1 + m], 0, 0, 0);
                    acc[1 + m] = __builtin_amdgcn_mfma_f32_16x16x32_f16(Sl, Vh[m][t], acc[1 + m], 0, 0, 0);
                    acc[1 + m] = __builtin_amdgcn_mfma_f32_16x16x32_f16(Sa, Vo[m][t], acc[1 + m], 0, 0, 0);
                    acc[1 + m] = __builtin_amdgcn_mfma_f32_16x16x32_f16(Sa, Vh[m][t], acc[1 + m], 0, 0, 0);
                }
            }
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int jo = mt * 16 + 4 * q + r;
            const int a = lo + jo, b = s - a;
            const bool ok = jo < L;
            const float sl = sp[((ok && b > 0) ? jo + dl : ZR) * CS + kk];
            const float su = sp[((ok && a > 0) ? jo + dl - 1 : ZR) * CS + kk];
            const float f = lk_sig(__builtin_fmaf(acc[0][r], us[0], accx[0][r]));
            const float lam = lk_sig(__builtin_fmaf(acc[1][r], us[1], accx[1][r]));
            const float o1 = lk_sig(__builtin_fmaf(acc[2][r], us[2], accx[2][r]));
            const float o2 = lk_sig(__builtin_fmaf(acc[3][r], us[3], accx[3][r]));
            const float gg = ftanh(__builtin_fmaf(acc[4][r], us[4], accx[4][r]));
            const float sbar = __builtin_fmaf(lam, sl - su, su);
            const float sv = __builtin_fmaf(f, sbar - gg, gg);
            const float hv = __builtin_fmaf(o1, ftanh(sv), o2 * sv);
            {
                const int wr = ok ? jo : XR;
                sc[wr * CS + kk] = sv;
                _Float16 hh, hl, sh, sl16;
                split16(hv * kHS6, hh, hl);
                split16(sv * kHS6, sh, sl16);
                _Float16* rw = reinterpret_cast<_Float16*>(hc + wr * (RSH * 2));
                rw[kk] = hh;
                rw[H + kk] = hl;
                rw[2 * H + kk] = sh;
                rw[3 * H + kk] = sl16;
            }
            const int el = (st + jo) * H + kk;
            const int ho = ok ? ((F.y(a) * D.Wc + F.x(b)) * H + kk) * 4 : kOOB6;
            bst(hv, rH, ho);
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, f32x4{f, lam, o1, o2}), rS4,
                                                   ok ? el * 16 : kOOB6, 0, 0);
            __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, f32x2{gg, sv}), rS2, ok ? el * 8 : kOOB6,
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

// Reverse wavefront: the quantities and the stash / dA layouts of k_bwd_leaky. For cell (a, b) with
// successors R = (a, b+1), D = (a+1, b) on the later diagonal:
//     dh    = dy + da(R).Ul^T + da(D).Uu^T
//     ds_in = ds_l(R) + ds_u(D) + da3(R).Vl^T + da3(D).Vu^T      (da3: the lam, o1, o2 columns)
template <int H>
__global__ __launch_bounds__(LK16<H>::MAXT) void k_bwd_leaky16(Dev D, int NT, const float* __restrict__ Ul,
                                                             const float* __restrict__ Uu,
                                                             const float* __restrict__ Vl,
                                                             const float* __restrict__ Vu,
                                                             const float* __restrict__ stash,
                                                             const float* __restrict__ dy_flat,
                                                             const float* __restrict__ dh_dirs,
                                                             float* __restrict__ dA, int32_t* __restrict__ done) {
    using Sh = LK16<H>;
    constexpr int NB = Sh::NB, KU = Sh::KU, KV = Sh::KV, RGB = Sh::RGB, RD = Sh::RD, G = Sh::G, G3 = Sh::G3;
    const int u = D.units[blockIdx.x];
    const int e = u >> 2, d = u & 3;
    const Flip F{D.rect[4 * e], D.rect[4 * e + 1], D.rect[4 * e + 2], D.rect[4 * e + 3], (d & 2) != 0, (d & 1) != 0};
    const int h = F.h, w = F.w;
    const int ry0 = D.real[4 * e], rx0 = D.real[4 * e + 1], rh = D.real[4 * e + 2], rw = D.real[4 * e + 3];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int mt = wave / NB, kb = wave % NB;
    const int col = lane & 15, q = lane >> 4;
    const int kk = kb * 16 + col;

    // B pieces: lane holds K rows 32 t + 8 q .. + 7 of column kk of [Ul^T; Uu^T] and of [Vl^T; Vu^T]
    u32x4 BU[KU][3], BV[KV][3];
#pragma unroll
    for (int t = 0; t < KU; ++t) {
        float v[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int n = 32 * t + 8 * q + i;
            v[i] = n < G ? Ul[((int64_t)d * H + kk) * G + n] : Uu[((int64_t)d * H + kk) * G + n - G];
        }
        split3b(v, BU[t]);
    }
#pragma unroll
    for (int t = 0; t < KV; ++t) {
        float v[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int n = 32 * t + 8 * q + i;
            v[i] = n < G3 ? Vl[((int64_t)d * H + kk) * G3 + n]
                          : (n < 2 * G3 ? Vu[((int64_t)d * H + kk) * G3 + n - G3] : 0.f);
        }
        split3b(v, BV[t]);
    }

    // LDS, two buffers each: rows of the bf16 pieces of a diagonal's gate gradients (piece p of gate g, unit k
    // at p G + g H + k), of ds sent to the left predecessor, and of ds sent to the upper one; row j is
    // diagonal position j, row ZR zeros, row XR takes the writes of lanes without a cell (no branch in a step)
    extern __shared__ __align__(16) unsigned char smem[];
    const int ZR = 16 * NT, XR = ZR + 1, ROWS = ZR + 2;
    const int ABUF = ROWS * RGB * 2, DBUF = ROWS * RD * 4;
    {
        uint32_t* z32 = reinterpret_cast<uint32_t*>(smem);
        for (int i = threadIdx.x; i < (2 * ABUF + 4 * DBUF) / 4; i += blockDim.x) z32[i] = 0u;
    }

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
            const int jo = mt * 16 + 4 * q + r;
            const bool ok = jo < L;
            const int a = lo + jo, b = s - a;
            const int ei = (st + jo) * H + kk;
            const int so4 = ok ? ei * 16 : kOOB6, so2 = ok ? ei * 8 : kOOB6;
            const f32x4 g4 = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rS4, so4, 0, 0));
            const f32x2 g2 = __builtin_bit_cast(f32x2, __builtin_amdgcn_raw_buffer_load_b64(rS2, so2, 0, 0));
            v[0][r] = g4[0]; v[1][r] = g4[1]; v[2][r] = g4[2]; v[3][r] = g4[3];
            v[4][r] = g2[0]; v[5][r] = g2[1];
            v[6][r] = bld(rS2, (ok && b > 0) ? (((stp + a - lop) * H + kk) * 2 + 1) * 4 : kOOB6);
            v[7][r] = bld(rS2, (ok && a > 0) ? (((stp + a - 1 - lop) * H + kk) * 2 + 1) * 4 : kOOB6);
            const int y = F.y(a), x = F.x(b);
            const int ly = y - ry0, lx = x - rx0;
            int uo = kOOB6;
            if (ok && per_dir) uo = ((y * D.Wc + x) * H + kk) * 4;
            if (ok && !per_dir && ly >= 0 && lx >= 0 && ly < rh && lx < rw) uo = ((ly * rw + lx) * H + kk) * 4;
            v[8][r] = bld(rU, uo);
        }
    };

    // the six terms of order <= 2^-16 of one K block, smallest first
    auto terms6 = [&](const u32x4 (&A)[3], const u32x4 (&B)[3], f32x4 c) {
        c = mfma_bf(A[2], B[0], c);
        c = mfma_bf(A[1], B[1], c);
        c = mfma_bf(A[0], B[2], c);
        c = mfma_bf(A[1], B[0], c);
        c = mfma_bf(A[0], B[1], c);
        return mfma_bf(A[0], B[0], c);
    };

    auto step = [&](int s, const float (&vc)[9][4], float (&vn)[9][4]) {
        const int L = dg_len(h, w, s), lo = dg_lo(h, w, s);
        const int st = (int)dg_start(h, w, s);
        const int lon = s + 1 < S ? dg_lo(h, w, s + 1) : 0;
        load_v(s - 1, vn);  // prefetch; consumed next step
        const unsigned char* ar = smem + ((s + 1) & 1) * ABUF;
        const float* dslr = reinterpret_cast<const float*>(smem + 2 * ABUF + ((s + 1) & 1) * DBUF);
        const float* dsur = reinterpret_cast<const float*>(smem + 2 * ABUF + 2 * DBUF + ((s + 1) & 1) * DBUF);
        unsigned char* aw = smem + (s & 1) * ABUF;
        float* dslw = reinterpret_cast<float*>(smem + 2 * ABUF + (s & 1) * DBUF);
        float* dsuw = reinterpret_cast<float*>(smem + 2 * ABUF + 2 * DBUF + (s & 1) * DBUF);
        f32x4 ah = f32x4{vc[8][0], vc[8][1], vc[8][2], vc[8][3]};
        f32x4 ah2 = f32x4{0.f, 0.f, 0.f, 0.f}, as = ah2, as2 = ah2;
        {
            const int j = mt * 16 + col;
            const int a = lo + j, b = s - a;
            const int jr = (j < L && b + 1 < w) ? a - lon : ZR;      // right successor (a, b+1)
            const int jd = (j < L && a + 1 < h) ? a + 1 - lon : ZR;  // lower successor (a+1, b)
            auto rd = [&](int row, int off, u32x4 (&A)[3]) {
                const unsigned char* p = ar + row * (RGB * 2) + off * 2;
#pragma unroll
                for (int k = 0; k < 3; ++k)
                    A[k] = *reinterpret_cast<const u32x4*>(__builtin_assume_aligned(p + k * (G * 2), 16));
            };
#pragma unroll
            for (int t = 0; t < KU; ++t) {
                const int k0 = 32 * t + 8 * q;
                u32x4 A[3];
                rd(k0 < G ? jr : jd, k0 < G ? k0 : k0 - G, A);
                if (t & 1) ah2 = terms6(A, BU[t], ah2);
                else ah = terms6(A, BU[t], ah);
            }
#pragma unroll
            for (int t = 0; t < KV; ++t) {
                const int k0 = 32 * t + 8 * q;
                u32x4 A[3];
                rd(k0 < G3 ? jr : (k0 < 2 * G3 ? jd : ZR), H + (k0 < G3 ? k0 : (k0 < 2 * G3 ? k0 - G3 : 0)), A);
                if (t & 1) as2 = terms6(A, BV[t], as2);
                else as = terms6(A, BV[t], as);
            }
            ah += ah2;
            as += as2;
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int jo = mt * 16 + 4 * q + r;
            const int a = lo + jo, b = s - a;
            const bool ok = jo < L;
            const float dsin = as[r] + dslr[((ok && b + 1 < w) ? a - lon : ZR) * RD + kk] +
                               dsur[((ok && a + 1 < h) ? a + 1 - lon : ZR) * RD + kk];
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
            {
                const int wr = ok ? jo : XR;
                uint16_t* rp = reinterpret_cast<uint16_t*>(aw + wr * (RGB * 2));
                const float dv[5] = {d0, d1, d2, d3, d4};
#pragma unroll
                for (int g = 0; g < 5; ++g) {
                    uint16_t p0, p1, p2;
                    split3b1(dv[g], p0, p1, p2);
                    rp[g * H + kk] = p0;
                    rp[G + g * H + kk] = p1;
                    rp[2 * G + g * H + kk] = p2;
                }
                dslw[wr * RD + kk] = dsbar * lam;
                dsuw[wr * RD + kk] = dsbar - dsbar * lam;
            }
            const int ea = (st + jo) * H + kk;
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, f32x4{d0, d1, d2, d3}), rA4,
                                                   ok ? ea * 16 : kOOB6, 0, 0);
            bst(d4, rA1, ok ? ea * 4 : kOOB6);
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
    // The unit is done: once every wave's gate-gradient stores are visible device-wide, flag it (the weight
    // gradient may then start on this direction of the example's cells while other units still run).
    if (done != nullptr) {
        __threadfence();
        __syncthreads();
        if (threadIdx.x == 0) __hip_atomic_store(done + u, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    }
}

typedef void (*FwdL16K)(Dev, const void*, int, int, const float*, const float*, const float*, const float*,
                        const float*, const float*, float*, float*);
typedef void (*BwdL16K)(Dev, int, const float*, const float*, const float*, const float*, const float*,
                        const float*, const float*, float*, int32_t*);

struct L16Entry {
    int H;
    FwdL16K fwd[4][2];  // [K steps of input channels - 1][f32, bf16 input]
    BwdL16K bwd;
    int NB, MAXT, RSH, CS, RGB, RD;
};
#define MDL_L16F(h, kx) {k_fwd_leaky16<h, kx, false>, k_fwd_leaky16<h, kx, true>}
#define MDL_L16(h)                                                                                             \
    {h, {MDL_L16F(h, 1), MDL_L16F(h, 2), MDL_L16F(h, 3), MDL_L16F(h, 4)}, k_bwd_leaky16<h>, LK16<h>::NB,        \
     LK16<h>::MAXT, LK16<h>::RSH, LK16<h>::CS, LK16<h>::RGB, LK16<h>::RD}
const L16Entry kL16[] = {MDL_L16(16), MDL_L16(32)};
#undef MDL_L16
#undef MDL_L16F

const L16Entry* l16_entry(int H) {
    for (const auto& m : kL16)
        if (m.H == H) return &m;
    return nullptr;
}

constexpr size_t kLdsMax16 = 160 * 1024;  // LDS of one workgroup on gfx950

int l16_tiles(int Lmax) { return (Lmax + 15) / 16; }

size_t l16_fwd_bytes(const L16Entry& m, int Lmax) {
    return 2 * (size_t)(16 * l16_tiles(Lmax) + 2) * ((size_t)m.RSH * 2 + (size_t)m.CS * 4);
}
size_t l16_bwd_bytes(const L16Entry& m, int Lmax) {
    return 2 * (size_t)(16 * l16_tiles(Lmax) + 2) * ((size_t)m.RGB * 2 + 2 * (size_t)m.RD * 4);
}

}  // namespace

// The matrix-core kernels take a layout when the hidden size is 16 or 32, the widest diagonal's tiles fit the
// workgroup and both wavefronts' LDS fits; the fp32 kernels of k_leaky.hip take every other one.
bool leaky16_used(int H, int Lmax) {
    const L16Entry* m = l16_entry(H);
    return m && 64 * l16_tiles(Lmax) * m->NB <= m->MAXT && l16_fwd_bytes(*m, Lmax) <= kLdsMax16 &&
           l16_bwd_bytes(*m, Lmax) <= kLdsMax16;
}

size_t leaky16_fwd_lds(int H, int Lmax) { return l16_fwd_bytes(*l16_entry(H), Lmax); }
size_t leaky16_bwd_lds(int H, int Lmax) { return l16_bwd_bytes(*l16_entry(H), Lmax); }

hipError_t launch_fwd_leaky16(const Dev& D, const void* x_canvas, int dtype, int C, int H, const float* Wx,
                              const float* b, const float* Ul, const float* Uu, const float* Vl, const float* Vu,
                              float* stash, float* h_dirs, hipStream_t st) {
    if (!leaky16_used(H, D.max_diag) || C < 1 || C > 4 * kMaxKX6) return hipErrorInvalidValue;
    const L16Entry* m = l16_entry(H);
    const int NT = l16_tiles(D.max_diag);
    launch(m->fwd[(C + 3) / 4 - 1][dtype != 0 ? 1 : 0], dim3(4 * D.n), dim3(64 * NT * m->NB), l16_fwd_bytes(*m, D.max_diag), st, D,
           x_canvas, C, NT, Wx, b, Ul, Uu, Vl, Vu, stash, h_dirs);
    return hipGetLastError();
}

hipError_t launch_bwd_leaky16(const Dev& D, int H, const float* Ul, const float* Uu, const float* Vl,
                              const float* Vu, const float* stash, const float* dy_flat, const float* dh_dirs,
                              float* dA, int32_t* done, hipStream_t st) {
    if (!leaky16_used(H, D.max_diag)) return hipErrorInvalidValue;
    const L16Entry* m = l16_entry(H);
    const int NT = l16_tiles(D.max_diag);
    launch(m->bwd, dim3(4 * D.n), dim3(64 * NT * m->NB), l16_bwd_bytes(*m, D.max_diag), st, D, NT, Ul, Uu, Vl, Vu,
           stash, dy_flat, dh_dirs, dA, done);
    return hipGetLastError();
}

}  // namespace mdl
