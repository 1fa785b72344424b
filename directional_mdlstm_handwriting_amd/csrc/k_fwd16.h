// k_fwd16.h — forward wavefront with the recurrent product on the f16 matrix cores.
//
// Same schedule as the other wavefront kernels ("No Padding Please" §IV-A and
// RETURNN §4.2: all cells of a local anti-diagonal are independent; one
// workgroup per (example, direction) unit walks its diagonals in order), but
// the recurrent product
//     a(cell) = Z(cell) + [h_left, h_up](cell) . [Ul; Uu]
// runs on v_mfma_f32_16x16x32_f16, which moves 8x the multiply-adds per
// cycle of the fp32 matrix instruction. h is split into an f16 pair
// h = hi + lo (about 22 bits), the weights into three f16 pieces
// U = hi + lo + r (r, the rounding residue of the pair, makes the weights
// exact to about 2^-33), and the product keeps the four terms
// h_hi.r + h_lo.U_hi + h_hi.U_lo + h_hi.U_hi, accumulated in fp32 in that
// order (smallest first), at 4 f16 instructions per 32-wide K block instead of
// 8 fp32 ones. Dropping r (a pair holds U only to about 2^-22 of each weight)
// perturbs every weight by a fixed amount in every cell, an error that the
// long chains of the recurrence accumulate coherently: on long word-like
// chains that alone put the outputs and gradients about twice as far from
// the exact result as plain fp32 evaluations are (measured against the
// float64 oracle with a float32 emulation of this arithmetic). The terms
// dropped now (h_lo times U_lo and r) are below 2^-21 of a product and vary
// from cell to cell, as fp32 rounding does. At H = 50 the residue's registers
// would spill, so that shape (short chains only: the third level of the stack)
// keeps the pair. f16 has a narrow exponent range, so
// h (|h| < 1) is scaled by 2^14 and each weight column by its own power of
// two (its largest magnitude lands in [2^14, 2^15)); the accumulator is scaled
// back exactly before x.Wx + b is added.
//
// The input projection x.Wx + b ("No Padding Please" §IV-B: the input-only
// part of the gates is one 1x1 convolution) is computed in the same step on
// the fp32 matrix cores (v_mfma_f32_16x16x4_f32, K = 4 channels per
// instruction, the bias seeding the accumulator), from the canvas pixels of
// the diagonal's cells: no projection tensor is written or read.
//
// Work split: NB * CG waves; wave = (16-wide block kb of hidden units, cell
// group cg). Cells of the diagonal are dealt round-robin to the CG cell
// groups, and inside a wave cell i sits in MFMA row 4*(i%4) + i/4, so that a
// lane's four accumulator rows hold cells q, q+4, q+8, q+12 (q = lane/16): a
// wave whose group has m cells on the widest diagonal needs NR = ceil(m/4)
// accumulator rows. NR is fixed per launch, so every step is one straight
// instruction sequence: the compiler then knows how many memory operations
// are in flight and waits for a prefetch with vmcnt(N) instead of draining
// every store (loads and stores retire in order on this architecture). The
// input pixels are prefetched three diagonals ahead into four register sets.
// The previous diagonal's h (as scaled f16 hi/lo) and c sit in LDS ping-pong
// buffers with a zero row standing in for a missing predecessor.
#pragma once

#include "kernels.h"
#include "devmath.h"

#include <type_traits>

namespace mdl {
namespace f16k {


constexpr int kOOB = 0x40000000;    // byte offset past every per-unit range used here (1 GiB)
constexpr float kHScale = 16384.f;  // 2^14: h in (-1, 1) -> f16 range
constexpr int kZD = 3;              // diagonals of input prefetch ahead
// The sigmoid gates take their argument in base-2 exponent form, sigmoid(a) = 1 / (1 + 2^(-a log2 e)): the
// factor -log2 e of gates i, f_l, f_u, o is folded into the weight scales and the bias, so their
// accumulators already hold the exponents. The cell input g = tanh(a) keeps its plain argument: tanh goes
// through ftanh, whose error is relative also near 0 (a small g or c would otherwise carry an absolute
// error of about 1e-7 into every gradient that multiplies it).
constexpr float kL2E = 1.44269504088896341f;
__host__ __device__ constexpr float gate_fold(int g) { return g < 4 ? -kL2E : 1.0f; }
__device__ inline float sig_e2(float t) { return frcp(1.0f + __builtin_amdgcn_exp2f(t)); }

template <int H>
struct F16Shape {
    static constexpr int NB = (H + 15) / 16;       // blocks of 16 hidden units
    static constexpr int HP = (H + 7) / 8 * 8;     // h_left / h_up segment in the K dimension
    static constexpr int KB = (2 * HP + 31) / 32;  // K blocks of 32
    static constexpr bool R3 = NB <= 2;            // weights as three f16 pieces (registers allow it)
    static_assert(NB <= 4, "hidden size above 64");
};

template <int N>
using IC = std::integral_constant<int, N>;

// KX: K steps of 4 input channels; BF16: canvas pixels stored as bf16
template <int H, int CG, int NR, int KX, bool BF16>
__global__ __launch_bounds__(64 * F16Shape<H>::NB * CG) void k_fwd16(Dev D, const void* __restrict__ xc, int C,
                                                                     const float* __restrict__ Wx,
                                                                     const float* __restrict__ bias,
                                                                     const float* __restrict__ Ul,
                                                                     const float* __restrict__ Uu,
                                                                     float* __restrict__ stash,
                                                                     float* __restrict__ hdirs,
                                                                     int32_t* __restrict__ done) {
    using Sh = F16Shape<H>;
    constexpr int HP = Sh::HP, KB = Sh::KB;
    constexpr bool R3 = Sh::R3;
    constexpr int G = 5 * H;
    const int u = D.units[blockIdx.x];
    const int e = u >> 2, d = u & 3;
    const int y0 = D.rect[4 * e], x0 = D.rect[4 * e + 1], h = D.rect[4 * e + 2], w = D.rect[4 * e + 3];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int kb = wave / CG, cg = wave % CG;
    const int q = lane >> 4, col = lane & 15;
    const int kk = kb * 16 + col;  // this lane's hidden unit (output column)
    const bool kok = kk < H;
    const int kc = kok ? kk : 0;

    // B operand: lane holds rows 32t + 8q .. +7 of column g*H + kk of [Ul; Uu] (Ul row k at K index k,
    // Uu row k at HP + k, zeros elsewhere), scaled per column by 2^E and split into f16 hi + lo + r.
    f16x8 Bh[5][KB], Bl[5][KB], Br[5][R3 ? KB : 1];
    float us[5];  // 2^-(E + 14) times the gate's fold: undoes both scalings
#pragma unroll
    for (int g = 0; g < 5; ++g) {
        float v[KB][8];
        float m = 0.f;
#pragma unroll
        for (int t = 0; t < KB; ++t)
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int k = 32 * t + 8 * q + i;
                float x = 0.f;
                if (kok) {
                    if (k < H) x = Ul[((int64_t)d * H + k) * G + g * H + kk];
                    else if (k >= HP && k - HP < H) x = Uu[((int64_t)d * H + (k - HP)) * G + g * H + kk];
                }
                v[t][i] = x;
                m = fmaxf(m, fabsf(x));
            }
        m = fmaxf(m, __shfl_xor(m, 16));
        m = fmaxf(m, __shfl_xor(m, 32));
        int E = 0;
        if (m > 0.f) {
            E = 14 - ((int)((__float_as_uint(m) >> 23) & 255) - 127);
            E = E < -100 ? -100 : (E > 100 ? 100 : E);
        }
        us[g] = ldexpf(1.0f, -(E + 14)) * gate_fold(g);  // undoes both scalings, times the gate's fold
#pragma unroll
        for (int t = 0; t < KB; ++t)
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float vs = ldexpf(v[t][i], E);
                _Float16 hi, lo;
                split16(vs, hi, lo);
                Bh[g][t][i] = hi;
                Bl[g][t][i] = lo;
                // vs - hi and then - lo are exact in fp32 (each operand holds the leading bits of the other)
                if constexpr (R3) Br[g][t][i] = (_Float16)((vs - (float)hi) - (float)lo);
            }
    }

    // input projection: B = Wx[d][4 ks + q][g*H + kk] for K step ks; the bias seeds the accumulators
    float Bx[5][KX], bz[5];
#pragma unroll
    for (int g = 0; g < 5; ++g) {
        bz[g] = kok ? bias[(int64_t)d * G + g * H + kk] * gate_fold(g) : 0.f;
#pragma unroll
        for (int ks = 0; ks < KX; ++ks) {
            const int c = 4 * ks + q;
            Bx[g][ks] = (kok && c < C) ? Wx[((int64_t)d * C + c) * G + g * H + kk] * gate_fold(g) : 0.f;
        }
    }

    // LDS, two buffers (previous / current diagonal) of NRW rows each: h * 2^14 as f16 hi and lo (row
    // stride RS halves), then c (row stride CS floats). Diagonal position j is kept in row P(j) (below);
    // row ZR is zeros, row XR absorbs the writes of lanes without a cell.
    constexpr int RS = 2 * HP + 8, CS = H + 4;
    constexpr int NRW = 16 * CG + 2, ZR = 16 * CG, XR = 16 * CG + 1;
    constexpr int HBUF = NRW * RS * 2, CBUF = NRW * CS * 4;  // bytes of one h / c buffer
    extern __shared__ __align__(16) unsigned char smem[];
    {
        uint32_t* z32 = reinterpret_cast<uint32_t*>(smem);
        for (int i = threadIdx.x; i < (HBUF + CBUF) / 2; i += blockDim.x) z32[i] = 0u;
    }
    const int64_t base = (int64_t)d * D.T + D.cell_off[e];
    const int64_t cells = (int64_t)h * w;
    const int64_t o1 = z1_offset(D.T, H);
    constexpr int XB = BF16 ? 2 : 4;  // bytes per input value
    const __amdgpu_buffer_rsrc_t rX = rsrc(xc, (int64_t)D.Hc * D.Wc * C * XB);
    const __amdgpu_buffer_rsrc_t rS4 = rsrc(stash + base * 4 * H, cells * 16 * H);
    const __amdgpu_buffer_rsrc_t rS2 = rsrc(stash + o1 + base * 4 * H, cells * 16 * H);
    const __amdgpu_buffer_rsrc_t rH = rsrc(hdirs + (int64_t)d * D.Hc * D.Wc * H, (int64_t)D.Hc * D.Wc * H * 4);
    const int S = h + w - 1;

    // Cell j of a diagonal belongs to cell group j % CG and is cell i = j / CG of that group's wave,
    // computed in MFMA row 4(i%4) + i/4. Its LDS row P(j) = 16(j % CG) + 4(i%4) + i/4: the 16 lanes that
    // gather one K block of the A operand then read 16 consecutive rows, and the odd row stride (in
    // 16-byte units) puts them on distinct banks. Positions outside [0, 16 CG) map to the zero row.
    auto P = [&](int j) {
        if (j < 0 || j >= 16 * CG) return ZR;
        const int i = j / CG;
        return 16 * (j % CG) + 4 * (i & 3) + (i >> 2);
    };

    // Every address of the step loop is a per-lane constant plus a per-step scalar. Cell (a, b) of the
    // unit (b = s - a on diagonal s) sits at canvas (Y0 + SY a, X0 + SX b), so its h byte offset is
    // HB + a DA + s DS + 4 kk; a = lo + j for position j on the diagonal. On diagonal s the left
    // predecessor of position j is position j + dl of diagonal s - 1 and the upper one j + dl - 1, with
    // dl = 0 while s < w and 1 after.
    const int SY = (d & 2) ? -1 : 1, SX = (d & 1) ? -1 : 1;
    const int Y0 = (d & 2) ? y0 + h - 1 : y0, X0 = (d & 1) ? x0 + w - 1 : x0;
    const int H4 = 4 * H;
    const int DA = SY * D.Wc * H4 - SX * H4, DS = SX * H4;
    const int HB = (Y0 * D.Wc + X0) * H4;
    int jo[NR], vh[NR], ve[NR];  // per accumulator row r: diagonal position, h offset, stash element
    int owc[NR], owh[NR];        // LDS byte offsets of the row's own c and h entries (within a buffer)
    int opc[NR][3];              // LDS byte offsets of c at positions jo - 1, jo, jo + 1
#pragma unroll
    for (int r = 0; r < NR; ++r) {
        jo[r] = (4 * r + q) * CG + cg;
        vh[r] = jo[r] * DA + 4 * kk;
        ve[r] = jo[r] * H + kk;
        const int pw = 16 * cg + 4 * q + r;  // P(jo[r])
        // a lane without a hidden unit writes the discard row; a row of a position beyond the diagonal takes
        // whatever its lane computes, since no later step reads positions past its predecessor's length
        owc[r] = kok ? pw * CS * 4 + 4 * kc : XR * CS * 4 + 4 * kc;
        owh[r] = kok ? pw * RS * 2 + 2 * kc : XR * RS * 2 + 2 * kc;
#pragma unroll
        for (int m = 0; m < 3; ++m) opc[r][m] = P(jo[r] + m - 1) * CS * 4 + 4 * kc;
    }
    const int ozc = ZR * CS * 4 + 4 * kc;
    const int ja = (4 * (col & 3) + (col >> 2)) * CG + cg;  // diagonal position of this lane's A row
    // canvas input of the A row's cell: byte offset XBASE + a XA + s XS + vx[ks] (channel 4 ks + q)
    const int XA = (SY * D.Wc * C - SX * C) * XB, XS = SX * C * XB;
    const int XBASE = (Y0 * D.Wc + X0) * C * XB;
    int vx[KX];
    bool cx[KX];
#pragma unroll
    for (int ks = 0; ks < KX; ++ks) {
        vx[ks] = ja * XA + (4 * ks + q) * XB;
        cx[ks] = 4 * ks + q < C;
    }
    int oah[3];  // LDS byte offsets of the h rows at positions ja - 1, ja, ja + 1
#pragma unroll
    for (int m = 0; m < 3; ++m) oah[m] = P(ja + m - 1) * RS * 2;
    const int oza = ZR * RS * 2;

    auto diag_len = [&](int s) {
        const int lo = s > w - 1 ? s - (w - 1) : 0;
        const int hi = s < h - 1 ? s : h - 1;
        return s < S ? hi - lo + 1 : 0;
    };

    // input pixels of this lane's A-row cell on diagonal s1, one value per K step (0 where absent)
    auto load_x = [&](int s1, float (&xv)[KX]) {
        const int L1 = diag_len(s1);
        const int lo1 = s1 > w - 1 ? s1 - (w - 1) : 0;
        const int px = XBASE + lo1 * XA + s1 * XS;
        const bool va = ja < L1;
#pragma unroll
        for (int ks = 0; ks < KX; ++ks) {
            const int off = (va & cx[ks]) ? px + vx[ks] : kOOB;
            if constexpr (BF16)
                xv[ks] = __uint_as_float((uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rX, off, 0, 0) << 16);
            else
                xv[ks] = bld(rX, off);
        }
    };

    float xs[4][KX];
    int st = 0;  // stash index of the first cell of diagonal s
#pragma unroll
    for (int i = 0; i < kZD; ++i) load_x(i, xs[i]);
    // wait for the first sets here, once: the loop then starts with nothing in flight, the same state
    // for every diagonal, and the compiler's per-step waits only cover the kZD-step-old prefetch
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    __syncthreads();

    // input projection x.Wx + b of one diagonal's A-row cells on the fp32 matrix cores, the bias seeding the
    // accumulators. It does not depend on the recurrence, so each step forms the next diagonal's projection
    // after its own gate arithmetic, while the matrix cores are otherwise idle: the step's dependent matrix
    // phase then holds only the recurrent product.
    f32x4 accx[5];
    auto project = [&](const float (&xv)[KX]) {
#pragma unroll
        for (int g = 0; g < 5; ++g) accx[g] = f32x4{bz[g], bz[g], bz[g], bz[g]};
#pragma unroll
        for (int ks = 0; ks < KX; ++ks)
#pragma unroll
            for (int g = 0; g < 5; ++g)
                accx[g] = __builtin_amdgcn_mfma_f32_16x16x4f32(xv[ks], Bx[g][ks], accx[g], 0, 0, 0);
    };
    project(xs[0]);

    // diagonal s at position POS = s mod 4 of the unrolled loop: buffer s & 1 is written and 1 - (s & 1)
    // read; at the end of the step input set (POS + 1) mod 4 feeds the projection of diagonal s + 1 and set
    // (POS + kZD) mod 4, whose diagonal s - 1 is done with, is refilled for diagonal s + kZD
    auto step = [&](int s, auto POSc) {
        constexpr int POS = decltype(POSc)::value;
        constexpr int CB = POS & 1;
        const int L = diag_len(s);
        const bool dl = s >= w;
        const int lo = dl ? s - (w - 1) : 0;
        const int Ml = L < s - lo ? L : s - lo;  // position j has a left predecessor iff j < Ml
        const int Tu = dl ? 0 : 1;                // ... and an upper one iff Tu <= j < L
        const unsigned char* hsp = smem + (1 - CB) * HBUF;
        const unsigned char* csp = smem + 2 * HBUF + (1 - CB) * CBUF;
        const int al = dl ? oah[2] : oah[1], au = dl ? oah[1] : oah[0];
        const int rl = ja < Ml ? al : oza;
        const int ru = (ja >= Tu && ja < L) ? au : oza;
        f16x8 Ah[KB], Al[KB];
#pragma unroll
        for (int t = 0; t < KB; ++t) {
            const int k0 = 32 * t + 8 * q;
            const int row = k0 < HP ? rl : (k0 < 2 * HP ? ru : oza);
            const int off = 2 * (k0 < HP ? k0 : (k0 < 2 * HP ? k0 - HP : 0));
            const unsigned char* p = hsp + row + off;
            Ah[t] = *reinterpret_cast<const f16x8*>(__builtin_assume_aligned(p, 16));
            Al[t] = *reinterpret_cast<const f16x8*>(__builtin_assume_aligned(p + 2 * HP, 16));
        }
        float cl[NR], cu[NR];
#pragma unroll
        for (int r = 0; r < NR; ++r) {
            const int ol = dl ? opc[r][2] : opc[r][1], ou = dl ? opc[r][1] : opc[r][0];
            cl[r] = *reinterpret_cast<const float*>(csp + (jo[r] < Ml ? ol : ozc));
            cu[r] = *reinterpret_cast<const float*>(csp + ((jo[r] >= Tu && jo[r] < L) ? ou : ozc));
        }
        f32x4 acc[5];
#pragma unroll
        for (int g = 0; g < 5; ++g) acc[g] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int t = 0; t < KB; ++t)
#pragma unroll
            for (int g = 0; g < 5; ++g) {
                if constexpr (R3) acc[g] = __builtin_amdgcn_mfma_f32_16x16x32_f16(Ah[t], Br[g][t], acc[g], 0, 0, 0);
                acc[g] = __builtin_amdgcn_mfma_f32_16x16x32_f16(Al[t], Bh[g][t], acc[g], 0, 0, 0);
                acc[g] = __builtin_amdgcn_mfma_f32_16x16x32_f16(Ah[t], Bl[g][t], acc[g], 0, 0, 0);
                acc[g] = __builtin_amdgcn_mfma_f32_16x16x32_f16(Ah[t], Bh[g][t], acc[g], 0, 0, 0);
            }
        const int ph = HB + lo * DA + s * DS;  // h offset of diagonal position 0, minus 4 kk
        const int pe = st * H;                 // stash element of diagonal position 0
        unsigned char* cw = smem + 2 * HBUF + CB * CBUF;
        unsigned char* hw = smem + CB * HBUF;
#pragma unroll
        for (int r = 0; r < NR; ++r) {
            const bool ok = jo[r] < L && kok;
            const float ig = sig_e2(__builtin_fmaf(acc[0][r], us[0], accx[0][r]));
            const float fl = sig_e2(__builtin_fmaf(acc[1][r], us[1], accx[1][r]));
            const float fu = sig_e2(__builtin_fmaf(acc[2][r], us[2], accx[2][r]));
            const float og = sig_e2(__builtin_fmaf(acc[3][r], us[3], accx[3][r]));
            const float gg = ftanh(__builtin_fmaf(acc[4][r], us[4], accx[4][r]));
            const float c = __builtin_fmaf(fl, cl[r], __builtin_fmaf(fu, cu[r], ig * gg));
            const float tc = ftanh(c);
            const float hv = og * tc;
            *reinterpret_cast<float*>(cw + owc[r]) = c;
            _Float16 hh, hl;
            split16(hv * kHScale, hh, hl);
            _Float16* hp = reinterpret_cast<_Float16*>(hw + owh[r]);
            hp[0] = hh;
            hp[HP] = hl;
            bst(hv, rH, ok ? ph + vh[r] : kOOB);
            const int el = pe + ve[r];
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, f32x4{ig, fl, fu, og}), rS4,
                                                   ok ? el * 16 : kOOB, 0, 0);
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, f32x4{gg, tc, cl[r], cu[r]}), rS2,
                                                   ok ? el * 16 : kOOB, 0, 0);
        }
        project(xs[(POS + 1) & 3]);  // diagonal s + 1 (prefetched two steps ago)
        // refill the set just consumed with diagonal s + kZD; issued here, its address arithmetic stays off
        // the dependent path between the barrier and the recurrent product
        load_x(s + kZD, xs[(POS + kZD) & 3]);
        st += L;
        __syncthreads();
    };
    int s = 0;
    for (; s + 4 <= S; s += 4) {
        step(s, IC<0>{});
        step(s + 1, IC<1>{});
        step(s + 2, IC<2>{});
        step(s + 3, IC<3>{});
    }
    if (s < S) step(s, IC<0>{});
    if (s + 1 < S) step(s + 1, IC<1>{});
    if (s + 2 < S) step(s + 2, IC<2>{});
    // the unit's h plane is complete: once every wave's stores are visible device-wide, flag it (the direction
    // sum may then start on the example while other units still run)
    if (done != nullptr) {
        __threadfence();
        __syncthreads();
        if (threadIdx.x == 0) __hip_atomic_store(done + u, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    }

    // h outside every computed region reads zero: the second half of the launch order (the smallest units,
    // done first) clears it, one band of canvas rows per workgroup, while the larger units still run
    // (a layout whose computed regions fill the canvas, as the padded stack does, has nothing to clear)
    const int half = (int)gridDim.x / 2, zb = (int)blockIdx.x - half, nz = (int)gridDim.x - half;
    const int64_t npx = (int64_t)D.Hc * D.Wc;
    if (zb >= 0 && D.T < npx) {
        const int64_t p0 = (int64_t)D.Hc * zb / nz * D.Wc, p1 = (int64_t)D.Hc * (zb + 1) / nz * D.Wc;
        const int64_t plane = npx * H;
        for (int64_t p = p0 + threadIdx.x; p < p1; p += blockDim.x) {
            if (D.eid[p] >= 0) continue;
            float* q = hdirs + p * H;
#pragma unroll
            for (int d4 = 0; d4 < 4; ++d4)
#pragma unroll
                for (int k = 0; k < H; ++k) q[d4 * plane + k] = 0.f;
        }
    }
}

typedef void (*Fwd16Kernel)(Dev, const void*, int, const float*, const float*, const float*, const float*, float*,
                            float*, int32_t*);

// one instantiated (hidden size, input K steps, bf16 input, cell groups CG) shape, with its kernels for
// NR = 1..4 accumulator rows; the widest diagonal must fit 16 CG cells
struct F16Entry {
    int H, KX;
    bool bf16;
    int CG, NB, HP;
    Fwd16Kernel fwd[4];
};
#define MDL_F16(h, kx, bf, cg)                                                                                \
    {h, kx, bf, cg, F16Shape<h>::NB, F16Shape<h>::HP,                                                         \
     {k_fwd16<h, cg, 1, kx, bf>, k_fwd16<h, cg, 2, kx, bf>, k_fwd16<h, cg, 3, kx, bf>, k_fwd16<h, cg, 4, kx, bf>}}
// the hidden-size-32 shapes, built in a translation unit of their own (with the matrix-core accumulators
// in the accumulation registers, which their register count needs)
const F16Entry* f16_entries_h32(int& n);

}  // namespace f16k
}  // namespace mdl
