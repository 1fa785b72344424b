// k_bwd16.hip — reverse wavefront (2D BPTT) with the recurrent product on the f16 matrix cores.
//
// The backward pass visits each unit's diagonals in reverse ("Single Stream
// Parallelization of Generalized LSTM-Like RNNs on a GPU": back-propagation in
// reverse order of the forward dependencies; RETURNN §4.2 for the 2D case).
// For cell (a, b) on diagonal s, with da the gradient of its five gate
// pre-activations and its successors R = (a, b+1), D = (a+1, b) on s+1:
//     dh     = dy(a, b) + da(R) . Ul^T + da(D) . Uu^T
//     dc_in  = dc(R) f_l(R) + dc(D) f_u(D)
//     tc = tanh c;  dc = dc_in + dh o (1 - tc^2)
//     da = [dc g i(1-i), dc c_l f_l(1-f_l), dc c_u f_u(1-f_u), dh tc o(1-o), dc i (1-g^2)]
//
// The workgroup of one (example, direction) unit has two roles, each in a loop of its own (so each has the
// whole register file of its waves to itself); every step of diagonal s ends in two barriers.
//  Matrix waves (the first four, one per SIMD) hold the recurrent weights, split, in registers. Before the
//     first barrier they read the gate gradients da of the later diagonal s + 1 from LDS (all of the step's
//     A operand at once) and form for each of its cells m the products X(m) = da(m) Ul^T and
//     Y(m) = da(m) Uu^T on v_mfma_f32_16x16x32_f16: the parts of dh that m sends to its left and upper
//     predecessors. Both operands are split into f16 hi + lo pairs (three partial products summed in
//     fp32). Gate gradients have no bound, so each cell's row of da was scaled by the power of two that
//     brings its largest magnitude into [2^14, 2^15) before it was split; its exponent sits in LDS beside
//     it and the product is scaled back exactly. The K dimension orders da by (gate, hidden unit), the
//     order of the columns of Ul and Uu, 5H entries padded to a multiple of 32.
//  Element waves (the others) own fixed (diagonal position, hidden unit) elements. Before the first
//     barrier, while the products run, they form every factor of dc and da that depends on the forward
//     alone (o (1 - tc^2) and the five gate-derivative products) from the forward's stash, which holds the
//     gates, tc = tanh c and the predecessors' memory states c_l, c_u, and work out the step's addresses. After it, dh = dy + X(R) + Y(D)
//     and dc_in leave a few products, the cell's scale (a maximum over the lanes of its DPP rows), the split
//     into the LDS A rows of the next step, dc f_l and dc f_u for the earlier diagonal, and the store of da
//     for the weight gradients. Their stash and upstream-gradient reads are issued KPD diagonals ahead.
// Rows of the LDS A operand are permuted so the 16 lanes gathering one K block read 16 consecutive rows
// on distinct banks.
// An element thread owns hidden units m and m + HE/2 of its cell, so that each of its global loads and stores
// (one unit per instruction) covers one contiguous run of the cell's units across the lanes. In LDS the two
// units sit side by side: the K order of the A operand and of the weight rows, and the column order of X, Y
// and the dc rows, place unit k at 2 (k mod HE/2) + k div (HE/2) within each gate.
#include "kernels.h"
#include "devmath.h"

#include <type_traits>

namespace mdl {

namespace {

constexpr int kOOB = 0x40000000;  // byte offset past every per-unit range used here (1 GiB)
constexpr int kMatWaves = 4;      // the matrix role, one wave per SIMD

template <int H>
struct B16Shape {
    static constexpr int NB = (H + 15) / 16;        // blocks of 16 hidden units
    static constexpr int HE = 16 * NB;              // hidden units padded to whole DPP rows
    static constexpr int CG = kMatWaves / NB;       // cell groups of the matrix waves
    static constexpr int KP = (5 * H + 31) / 32 * 32;  // K extent of one cell's da: 5H, padded
    static constexpr int KT = KP / 32;              // K blocks of 32
    static_assert(NB <= 2, "hidden size above 32");
    static_assert(H % 16 == 0, "hidden size not a multiple of 16");
};

template <int N>
using IC = std::integral_constant<int, N>;

// LDS byte pointer (32-bit address); values of this type held across a barrier keep their fixed offsets
// foldable into the LDS instructions
typedef __attribute__((address_space(3))) unsigned char* lds_p;

// exact power-of-two scale 2^E that brings m (> 0) into [2^14, 2^15), clamped to [-100, 100] (for m = 0
// it is 100: a row of zeros stays zero under any scale)
__device__ inline int scale_exp(uint32_t mbits) {
    const int E = 141 - (int)((mbits >> 23) & 255);
    return E < -100 ? -100 : (E > 100 ? 100 : E);
}

// largest value of x over the 16 lanes of each row of the wave (DPP within rows)
// (0 is the identity of the maximum, so each lane move can fold into the max instruction)
__device__ inline uint32_t row16_max(uint32_t x) {
    x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0xB1, 0xF, 0xF, true));   // quad_perm [1,0,3,2]
    x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x4E, 0xF, 0xF, true));   // quad_perm [2,3,0,1]
    x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x124, 0xF, 0xF, true));  // row_ror:4
    x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x128, 0xF, 0xF, true));  // row_ror:8
    return x;
}
// ... over the 8 lanes of each half-row
__device__ inline uint32_t row8_max(uint32_t x) {
    x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0xB1, 0xF, 0xF, true));   // quad_perm [1,0,3,2]
    x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x4E, 0xF, 0xF, true));   // quad_perm [2,3,0,1]
    x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x141, 0xF, 0xF, true));  // row_half_mirror
    return x;
}

// f16 pair of a scaled value v (|v| < 2^15): hi is v with its low 13 mantissa bits cleared, which f16
// holds exactly (11 significant bits; below the f16 normal range the rounding is under 2^-25), and
// lo = v - hi rounded to f16, so hi + lo is v to about 2^-21 of |v|
__device__ inline float hi_part(float v) { return __uint_as_float(__float_as_uint(v) & 0xFFFFE000u); }

// NE unit pairs per element-wave thread, EW element waves (NE 64 EW covers the cells x padded unit pairs of
// the widest diagonal), KPD diagonals of prefetch ahead
template <int H, int NE, int EW, int KPD>
__global__ __launch_bounds__(64 * (kMatWaves + EW)) void k_bwd16(Dev D, const float* __restrict__ Ul,
                                                                 const float* __restrict__ Uu,
                                                                 const float* __restrict__ stash,
                                                                 const float* __restrict__ dy_flat,
                                                                 const float* __restrict__ dh_dirs,
                                                                 float* __restrict__ dA, int32_t* __restrict__ done) {
    using Sh = B16Shape<H>;
    constexpr int NB = Sh::NB, HE = Sh::HE, CG = Sh::CG, KP = Sh::KP, KT = Sh::KT, HP2 = HE / 2;
    constexpr int G = 5 * H;
    constexpr int NT = 64 * (kMatWaves + EW), ET = 64 * EW, NS = KPD + 1;
    const int u = D.units[blockIdx.x];
    const int e = u >> 2, d = u & 3;
    const int y0 = D.rect[4 * e], x0 = D.rect[4 * e + 1], h = D.rect[4 * e + 2], w = D.rect[4 * e + 3];
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;

    // LDS, two buffers (written on diagonals of even / odd distance from the last) of NRW rows: the scale
    // exponent (ints, one copy per lane of the cell so that no two lanes write one word), dc*f_l and dc*f_u (row
    // stride CS floats) and the split, scaled da as f16 [hi | lo][gate][unit] (each piece KP halves, row
    // stride RA); one buffer each of the products X and Y of the later diagonal (row stride CS). The small
    // buffers come first, where the 16-bit offsets of the LDS instructions reach them. Diagonal position j
    // lives in row P(j) (below); ZR is a zero row. Each cell group's
    // block of 16 rows is shifted by a further SK (A, exponents) or SKC (the float rows) bytes per group, so
    // that the cells of different groups that one wave writes together fall on different banks.
    constexpr int RA = 2 * KP + 8, CS = HE + 4;
    constexpr int NRW = 16 * CG + 1, ZR = 16 * CG;
    constexpr int SK = 128 / CG, SKC = NB == 1 ? 64 : 0, NBLK = NRW / 16 + 1;
    constexpr int ABUF = NRW * RA * 2 + NBLK * SK, EBUF = NRW * HP2 * 4 + NBLK * SK, CBUF = NRW * CS * 4 + NBLK * SKC;
    auto rowA = [](int r) { return r * RA * 2 + (r >> 4) * SK; };    // byte offsets of row r in a buffer
    auto rowE = [](int r) { return r * HP2 * 4 + (r >> 4) * SK; };
    auto rowC = [](int r) { return r * CS * 4 + (r >> 4) * SKC; };
    constexpr int OFF_E = 0, OFF_CL = OFF_E + 2 * EBUF, OFF_CU = OFF_CL + 2 * CBUF;
    constexpr int OFF_X = OFF_CU + 2 * CBUF, OFF_Y = OFF_X + CBUF, OFF_A = (OFF_Y + CBUF + 15) / 16 * 16;
    constexpr int LDS_BYTES = OFF_A + 2 * ABUF;
    extern __shared__ __align__(16) unsigned char smem[];
    {
        uint32_t* z32 = reinterpret_cast<uint32_t*>(smem);
        for (int i = tid; i < LDS_BYTES / 4; i += NT) z32[i] = 0u;
    }
    const int S = h + w - 1;

    // Cell j of a diagonal belongs to cell group j % CG and is cell i = j / CG of that group's matrix wave,
    // computed in MFMA row 4(i%4) + i/4; its LDS row P(j) = 16(j % CG) + 4(i%4) + i/4 makes the 16 lanes
    // that gather one K block read 16 consecutive rows. Positions outside [0, 16 CG) map to the zero row.
    auto P = [&](int j) {
        if (j < 0 || j >= 16 * CG) return ZR;
        const int i = j / CG;
        return 16 * (j % CG) + 4 * (i & 3) + (i >> 2);
    };
    auto diag_len = [&](int s) {
        if (s < 0 || s >= S) return 0;
        const int lo = s > w - 1 ? s - (w - 1) : 0;
        const int hi = s < h - 1 ? s : h - 1;
        return hi - lo + 1;
    };
    auto diag_lo = [&](int s) { return s > w - 1 ? s - (w - 1) : 0; };
    __syncthreads();

    if (wave < kMatWaves) {
        // ================= matrix role =================
        // output block kb, cell group cg; lane (q, col)
        const int kb = wave / CG, cg = wave % CG;
        const int q = lane >> 4, col = lane & 15;
        // A wave computes two output column blocks ("pairs") for its 16 cells: with one block of hidden
        // units, X and Y of that block; with two, blocks 0 and 1 of X (kb = 0) or of Y (kb = 1).
        // B operand of pair p: U^T rows in the K order of the A operand (gate-major; within a gate, unit k at
        // 2 (k mod HP2) + k div HP2): for K block t the lane holds K rows 32t + 8q + i, i < 8 (zero from 5H on).
        // Scaled per output column by 2^E and split into f16 hi + lo.
        auto pair_y = [&](int p) { return NB == 1 ? p : kb; };               // pair computes Y (uses Uu)
        auto pair_col = [&](int p) { return 16 * (NB == 1 ? 0 : p) + col; };  // output hidden unit
        f16x8 Bh[2][KT], Bl[2][KT];
        int ec[2];  // the columns' scale exponents, negated
#pragma unroll
        for (int pp = 0; pp < 2; ++pp) {
            float v[KT][8];
            float m = 0.f;
            const float* U = pair_y(pp) ? Uu : Ul;
            const int kc = pair_col(pp);
#pragma unroll
            for (int t = 0; t < KT; ++t)
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const int kk = 32 * t + 8 * q + i;
                    const int pk = kk % H;  // position within the gate
                    const int uk = kk - pk + (pk >> 1) + (pk & 1) * HP2;  // U column: (gate, unit)
                    float x = 0.f;
                    if (kk < G) x = U[((int64_t)d * H + kc) * G + uk];
                    v[t][i] = x;
                    m = fmaxf(m, fabsf(x));
                }
            m = fmaxf(m, __shfl_xor(m, 16));
            m = fmaxf(m, __shfl_xor(m, 32));
            const int E = scale_exp(__float_as_uint(m));
            ec[pp] = -E;
#pragma unroll
            for (int t = 0; t < KT; ++t)
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    _Float16 hi, lo;
                    split16(ldexpf(v[t][i], E), hi, lo);
                    Bh[pp][t][i] = hi;
                    Bl[pp][t][i] = lo;
                }
        }
        // The lane's A row is its own cell ja = (4 (col & 3) + (col >> 2)) CG + cg of the later diagonal; its
        // output rows r are the cells (4r + q) CG + cg, at LDS rows 16 cg + 4q + r, whose scale exponents the
        // product carries.
        const int oa1 = rowA(P((4 * (col & 3) + (col >> 2)) * CG + cg));
        const int orow = 16 * cg + 4 * q;
        for (int s = S - 1; s >= 0; --s) {
            const int CB = (S - 1 - s) & 1;  // buffer this step's gate gradients go to; 1 - CB holds s + 1's
            const unsigned char* ap = smem + OFF_A + (1 - CB) * ABUF + oa1;
            const unsigned char* ep = smem + OFF_E + (1 - CB) * EBUF;
            f16x8 ah[KT], al[KT];
#pragma unroll
            for (int t = 0; t < KT; ++t) {
                const unsigned char* p = ap + (32 * t + 8 * q) * 2;
                ah[t] = *reinterpret_cast<const f16x8*>(__builtin_assume_aligned(p, 16));
                al[t] = *reinterpret_cast<const f16x8*>(__builtin_assume_aligned(p + KP * 2, 16));
            }
            int er[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) er[r] = *reinterpret_cast<const int*>(ep + rowE(orow + r));
            f32x4 acc[2];
#pragma unroll
            for (int pp = 0; pp < 2; ++pp) acc[pp] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int t = 0; t < KT; ++t)
#pragma unroll
                for (int pp = 0; pp < 2; ++pp) {
                    acc[pp] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah[t], Bh[pp][t], acc[pp], 0, 0, 0);
                    acc[pp] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah[t], Bl[pp][t], acc[pp], 0, 0, 0);
                    acc[pp] = __builtin_amdgcn_mfma_f32_16x16x32_f16(al[t], Bh[pp][t], acc[pp], 0, 0, 0);
                }
            // every LDS read of the step ahead of the products: the reads then overlap one another, and the
            // products wait only for the operands they take
            __builtin_amdgcn_sched_group_barrier(0x100, 2 * KT + 4, 0);  // LDS reads
            __builtin_amdgcn_sched_group_barrier(0x008, 6 * KT, 0);      // the products
            // output unit k goes to column 2 (k mod HP2) + k div HP2: with two blocks of units (both pairs
            // of one product) units col and 16 + col are one 8-byte word
            if constexpr (NB == 2) {
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    *reinterpret_cast<f32x2*>(smem + (kb ? OFF_Y : OFF_X) + rowC(orow + r) + col * 8) =
                        f32x2{ldexpf(acc[0][r], ec[0] - er[r]), ldexpf(acc[1][r], ec[1] - er[r])};
            } else {
                const int oc = (2 * (col % HP2) + col / HP2) * 4;
#pragma unroll
                for (int pp = 0; pp < 2; ++pp)
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        *reinterpret_cast<float*>(smem + (pp ? OFF_Y : OFF_X) + rowC(orow + r) + oc) =
                            ldexpf(acc[pp][r], ec[pp] - er[r]);
            }
            __syncthreads();  // X and Y of diagonal s + 1 are in LDS
            __syncthreads();  // the element waves have written diagonal s's gate gradients
        }
    } else {
    // ================= element role =================
    // Each thread owns NE pairs of hidden units (m, m + HP2) of one diagonal position: the HP2 lanes of a
    // cell sit in one DPP row (H = 32) or half-row (H = 16), each of its global accesses is one unit (the HP2
    // lanes of a cell read or write one contiguous run), and in LDS the pair is adjacent, so each gate's f16
    // pair goes to LDS as one 4-byte word.
    const int ry0 = D.real[4 * e], rx0 = D.real[4 * e + 1], rh = D.real[4 * e + 2], rw = D.real[4 * e + 3];
    const int et = tid - 64 * kMatWaves;
    const int64_t base = (int64_t)d * D.T + D.cell_off[e];
    const int64_t cells = (int64_t)h * w;
    const int64_t o1 = z1_offset(D.T, H);
    const __amdgpu_buffer_rsrc_t rS4 = rsrc(stash + base * 4 * H, cells * 16 * H);
    const __amdgpu_buffer_rsrc_t rS2 = rsrc(stash + o1 + base * 4 * H, cells * 16 * H);
    const __amdgpu_buffer_rsrc_t rA4 = rsrc(dA + base * 4 * H, cells * 16 * H);
    const __amdgpu_buffer_rsrc_t rA1 = rsrc(dA + o1 + base * H, cells * 4 * H);
    const bool per_dir = dh_dirs != nullptr;
    const __amdgpu_buffer_rsrc_t rU =
        per_dir ? rsrc(dh_dirs + (int64_t)d * D.Hc * D.Wc * H, (int64_t)D.Hc * D.Wc * H * 4)
                : rsrc(dy_flat + D.flat_off[e] * H, (int64_t)rh * rw * H * 4);

    // pair n of this thread is (position pj, units 2 pm, 2 pm + 1).
    // Cell (a, b) sits at canvas (Y0 + SY a, X0 + SX b). The upstream gradient's byte offset is
    // UB + a UA + s US + 4 k (b = s - a): on the canvas plane for a per-direction gradient, else in
    // the example's flat real-pixel block, where the cell must also lie in the real region.
    const int SY = (d & 2) ? -1 : 1, SX = (d & 1) ? -1 : 1;
    const int Y0 = (d & 2) ? y0 + h - 1 : y0, X0 = (d & 1) ? x0 + w - 1 : x0;
    const int H4 = 4 * H;
    const int rowlen = per_dir ? D.Wc : rw;
    const int UY = per_dir ? Y0 : Y0 - ry0, UX = per_dir ? X0 : X0 - rx0;
    const int UA = SY * rowlen * H4 - SX * H4, US = SX * H4;
    const int UB = (UY * rowlen + UX) * H4;
    // real region in unit coordinates: a in [ar0, ar1), b in [br0, br1)
    const int ar0 = (d & 2) ? h - (ry0 - y0) - rh : ry0 - y0, ar1 = ar0 + rh;
    const int br0 = (d & 1) ? w - (rx0 - x0) - rw : rx0 - x0, br1 = br0 + rw;
    int pj[NE], vu[NE], ve[NE];  // position; upstream-gradient and stash offsets of unit m (unit m + HP2 follows
                                 // at + 4 HP2 bytes and + HP2 elements)
    int wa[NE], we[NE], wc[NE];  // own LDS offsets (within a buffer)
    int oc[NE][3];               // LDS row offsets (stride CS) of positions pj - 1, pj, pj + 1
#pragma unroll
    for (int n = 0; n < NE; ++n) {
        const int el = et + ET * n;
        pj[n] = el / HP2;
        const int pm = el - pj[n] * HP2, k0 = 2 * pm;  // units pm, pm + HP2; LDS columns k0, k0 + 1
        vu[n] = pj[n] * UA + 4 * pm;
        ve[n] = pj[n] * H + pm;
        const int pr = P(pj[n]);
        wa[n] = rowA(pr) + 2 * k0;
        we[n] = rowE(pr) + 4 * pm;
        wc[n] = rowC(pr) + 4 * k0;
#pragma unroll
        for (int m = 0; m < 3; ++m) oc[n][m] = rowC(P(pj[n] + m - 1)) + 4 * k0;
    }
    // the forward's values of this thread's units on one diagonal (SA, SB; one unit each) and their
    // upstream gradient
    struct Fw {
        f32x4 fa[NE][2], fb[NE][2];
        f32x2 dy[NE];
    };
    // s1: diagonal, st1: stash index of its first cell
    auto load_f = [&](int s1, int st1, Fw& f) {
        const int L1 = diag_len(s1);
        const int lo1 = diag_lo(s1 < 0 ? 0 : s1);
        const int pe = st1 * H;
        const int pu0 = UB + lo1 * UA + s1 * US;
        // real-region bounds as position ranges: a = lo1 + j in [ar0, ar1), b = s1 - lo1 - j in [br0, br1)
        const int jr0 = max(ar0 - lo1, s1 - lo1 - br1 + 1), jr1 = min(ar1 - lo1, s1 - lo1 - br0 + 1);
#pragma unroll
        for (int n = 0; n < NE; ++n) {
            // predicates combined without short-circuit evaluation: plain selects, no branches
            const bool ok = pj[n] < L1;
            const int so = ok ? (pe + ve[n]) * 16 : kOOB;
#pragma unroll
            for (int u2 = 0; u2 < 2; ++u2) {
                f.fa[n][u2] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rS4, so + 16 * HP2 * u2, 0, 0));
                f.fb[n][u2] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rS2, so + 16 * HP2 * u2, 0, 0));
            }
            const bool vy = ok & (per_dir | ((pj[n] >= jr0) & (pj[n] < jr1)));
            const int uo = vy ? pu0 + vu[n] : kOOB;
#pragma unroll
            for (int u2 = 0; u2 < 2; ++u2)
                f.dy[n][u2] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rU, uo + 4 * HP2 * u2, 0, 0));
        }
    };

    Fw fs[NS];
    // stash index of the first cell of the prefetch diagonal s - KPD
    int stz = (int)cells - 1;  // diagonal S - 1 is the single last cell
#pragma unroll
    for (int i = 0; i < KPD; ++i) {
        load_f(S - 1 - i, stz, fs[i]);
        stz -= diag_len(S - 2 - i);
    }
    int st = (int)cells - 1;  // stash index of the first cell of diagonal s

    // diagonal s at position POS = (S - 1 - s) mod NS of the unrolled loop: prefetch set POS is consumed,
    // (POS + KPD) mod NS refilled; with NS even the LDS buffer parity (S - 1 - s) & 1 is POS & 1
    static_assert(NS % 2 == 0, "the unrolled loop must keep the buffer parity");
    typedef __attribute__((address_space(3))) f32x2 lds_f2;
    typedef __attribute__((address_space(3))) uint32_t lds_u32;
    auto step = [&](int s, auto POSc) {
        constexpr int POS = decltype(POSc)::value;
        constexpr int CB = POS & 1;
        load_f(s - KPD, stz, fs[(POS + KPD) % NS]);
        stz -= diag_len(s - KPD - 1);
        // ---- before the products are in: the factors into place, the step's addresses ----
        const Fw& f = fs[POS];
        const int L = diag_len(s);
        const int dn = s >= w - 1 ? 1 : 0;  // successors of position j: right j - dn, down j + 1 - dn
        const int pe = st * H;
        float cB[NE][2], c0[NE][2], c1[NE][2], c2[NE][2], c3[NE][2], c4[NE][2], dyv[NE][2], flv[NE][2],
            fuv[NE][2];
        lds_p rr[NE], rd[NE], oa[NE], oe[NE], ocw[NE];
        int og4[NE], og1[NE];
        const lds_p L0 = (lds_p)smem;
#pragma unroll
        for (int n = 0; n < NE; ++n) {
            const int j = pj[n];
            // successors' rows: right j - dn, lower j + 1 - dn. A position outside the later diagonal has a row
            // of zeros: the zero row below 0 and from 16 CG on, and in between the row its element wrote zeros to
            // (an element outside its diagonal computes exact zeros, its stash loads being masked) or, never
            // written, still holds the zeros of the start.
            rr[n] = L0 + (dn ? oc[n][0] : oc[n][1]);
            rd[n] = L0 + (dn ? oc[n][1] : oc[n][2]);
            const bool ok = j < L;
            oa[n] = L0 + wa[n] + CB * ABUF;
            oe[n] = L0 + we[n];
            ocw[n] = L0 + wc[n];
            const int el = pe + ve[n];
            og4[n] = ok ? el * 16 : kOOB;
            og1[n] = ok ? el * 4 : kOOB;
#pragma unroll
            for (int u2 = 0; u2 < 2; ++u2) {
                f32x4 ka, kb;
                bwd_factors(f.fa[n][u2], f.fb[n][u2], ka, kb);
                c0[n][u2] = ka[0];
                c1[n][u2] = ka[1];
                c2[n][u2] = ka[2];
                c3[n][u2] = ka[3];
                c4[n][u2] = kb[0];
                cB[n][u2] = kb[1];
                flv[n][u2] = kb[2];
                fuv[n][u2] = kb[3];
                dyv[n][u2] = f.dy[n][u2];
            }
        }
        // keep all of it before the barrier (the compiler would otherwise sink it into the part after)
#pragma unroll
        for (int n = 0; n < NE; ++n) {
#pragma unroll
            for (int u2 = 0; u2 < 2; ++u2) {
                asm volatile("" : "+v"(cB[n][u2]), "+v"(c0[n][u2]), "+v"(c1[n][u2]), "+v"(c2[n][u2]),
                             "+v"(c3[n][u2]), "+v"(c4[n][u2]));
                asm volatile("" : "+v"(dyv[n][u2]), "+v"(flv[n][u2]), "+v"(fuv[n][u2]));
            }
            asm volatile("" : "+v"(rr[n]), "+v"(rd[n]), "+v"(oa[n]), "+v"(oe[n]), "+v"(ocw[n]), "+v"(og4[n]),
                         "+v"(og1[n]));
        }
        __syncthreads();  // X and Y of diagonal s + 1 are in LDS
        // ---- the rest of dc and da: all LDS reads first, then the arithmetic, then the writes ----
        constexpr int RCL = OFF_CL + (1 - CB) * CBUF, RCU = OFF_CU + (1 - CB) * CBUF;  // the later diagonal's
        constexpr int WE = OFF_E + CB * EBUF, WCL = OFF_CL + CB * CBUF, WCU = OFF_CU + CB * CBUF;  // this one's
        f32x2 xv[NE], yv[NE], lv_[NE], uv[NE];
#pragma unroll
        for (int n = 0; n < NE; ++n) {
            xv[n] = *reinterpret_cast<lds_f2*>(rr[n] + OFF_X);
            yv[n] = *reinterpret_cast<lds_f2*>(rd[n] + OFF_Y);
            lv_[n] = *reinterpret_cast<lds_f2*>(rr[n] + RCL);
            uv[n] = *reinterpret_cast<lds_f2*>(rd[n] + RCU);
        }
        float dcv[NE][2], dd[NE][2][5];
        uint32_t mb[NE];
#pragma unroll
        for (int n = 0; n < NE; ++n) {
            float am = 0.f;
#pragma unroll
            for (int u2 = 0; u2 < 2; ++u2) {
                // dh: X of the right successor and Y of the lower one (zero rows when absent), plus dy
                const float dh = (xv[n][u2] + yv[n][u2]) + dyv[n][u2];
                const float dc = __builtin_fmaf(dh, cB[n][u2], lv_[n][u2] + uv[n][u2]);
                dcv[n][u2] = dc;
                dd[n][u2][0] = dc * c0[n][u2];
                dd[n][u2][1] = dc * c1[n][u2];
                dd[n][u2][2] = dc * c2[n][u2];
                dd[n][u2][3] = dh * c3[n][u2];
                dd[n][u2][4] = dc * c4[n][u2];
#pragma unroll
                for (int g = 0; g < 5; ++g) am = fmaxf(am, fabsf(dd[n][u2][g]));
            }
            // scale of this cell: the largest |da| over its lanes (non-negative floats order like their bits)
            mb[n] = __float_as_uint(am);
            // dc f_l and dc f_u for the earlier diagonal: written now, while the scale is worked out
            *reinterpret_cast<lds_f2*>(ocw[n] + WCL) = f32x2{dcv[n][0] * flv[n][0], dcv[n][1] * flv[n][1]};
            *reinterpret_cast<lds_f2*>(ocw[n] + WCU) = f32x2{dcv[n][0] * fuv[n][0], dcv[n][1] * fuv[n][1]};
        }
#pragma unroll
        for (int n = 0; n < NE; ++n) mb[n] = NB == 1 ? row8_max(mb[n]) : row16_max(mb[n]);
#pragma unroll
        for (int n = 0; n < NE; ++n) {
            const int E = scale_exp(mb[n]);
            float sv[2][5], tv[2][5];
#pragma unroll
            for (int u2 = 0; u2 < 2; ++u2)
#pragma unroll
                for (int g = 0; g < 5; ++g) {
                    sv[u2][g] = ldexpf(dd[n][u2][g], E);
                    tv[u2][g] = hi_part(sv[u2][g]);
                }
            // gate g of the thread's units goes to K = g H + k0, k0 + 1: one word per gate and piece
#pragma unroll
            for (int g = 0; g < 5; ++g) {
                const f16x2 hp = __builtin_convertvector((f32x2){tv[0][g], tv[1][g]}, f16x2);
                const f16x2 lp = __builtin_convertvector((f32x2){sv[0][g] - tv[0][g], sv[1][g] - tv[1][g]}, f16x2);
                *reinterpret_cast<lds_u32*>(oa[n] + OFF_A + 2 * g * H) = __builtin_bit_cast(uint32_t, hp);
                *reinterpret_cast<lds_u32*>(oa[n] + OFF_A + 2 * KP + 2 * g * H) = __builtin_bit_cast(uint32_t, lp);
            }
            *reinterpret_cast<lds_u32*>(oe[n] + WE) = (uint32_t)E;
#pragma unroll
            for (int u2 = 0; u2 < 2; ++u2)
                __builtin_amdgcn_raw_buffer_store_b128(
                    __builtin_bit_cast(u32x4, f32x4{dd[n][u2][0], dd[n][u2][1], dd[n][u2][2], dd[n][u2][3]}), rA4,
                    og4[n] + 16 * HP2 * u2, 0, 0);
#pragma unroll
            for (int u2 = 0; u2 < 2; ++u2)
                __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, dd[n][u2][4]), rA1,
                                                      og1[n] + 4 * HP2 * u2, 0, 0);
        }
        st -= diag_len(s - 1);
        __syncthreads();  // diagonal s's gate gradients are written
    };
    int s = S - 1;
    for (; s - (NS - 1) >= 0; s -= NS) {
        step(s, IC<0>{});
        step(s - 1, IC<1>{});
        step(s - 2, IC<2>{});
        if constexpr (NS > 3) step(s - 3, IC<3>{});
    }
    if (s >= 0) step(s, IC<0>{});
    if (s - 1 >= 0) step(s - 1, IC<1>{});
    if constexpr (NS > 3)
        if (s - 2 >= 0) step(s - 2, IC<2>{});
    }
    // The unit is done: once every wave's gate-gradient stores are visible device-wide, flag it (the weight
    // gradient may then start on this direction of the example's cells while other units still run).
    if (done != nullptr) {
        __threadfence();
        __syncthreads();
        if (tid == 0) __hip_atomic_store(done + u, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    }
}

typedef void (*Bwd16Kernel)(Dev, const float*, const float*, const float*, const float*, const float*, float*,
                            int32_t*);

// hidden sizes of the workloads, each with its (unit pairs per thread, element waves) shapes in order of
// preference: the smallest workgroup that covers the widest diagonal
struct B16Shape2 {
    int NE, EW;
    Bwd16Kernel k;
};
struct B16Entry {
    int H, NB, CG;
    B16Shape2 shapes[4];
};
#define MDL_B16S(h, ne, ew, pd) {ne, ew, k_bwd16<h, ne, ew, pd>}
const B16Entry kB16[] = {
    {16, B16Shape<16>::NB, B16Shape<16>::CG,
     {MDL_B16S(16, 1, 4, 3), MDL_B16S(16, 1, 8, 3), {0, 0, nullptr}, {0, 0, nullptr}}},
    {32, B16Shape<32>::NB, B16Shape<32>::CG,
     {MDL_B16S(32, 1, 4, 3), MDL_B16S(32, 1, 8, 3), {0, 0, nullptr}, {0, 0, nullptr}}}};
#undef MDL_B16S

// the widest diagonal must fit the matrix waves' tiles (16 CG cells) and one of the element shapes
const B16Shape2* b16_shape(const B16Entry& m, int Lmax) {
    const int elems = Lmax * 8 * m.NB;  // unit pairs
    for (const auto& sh : m.shapes)
        if (sh.k && elems <= sh.NE * 64 * sh.EW) return &sh;
    return nullptr;
}
const B16Entry* b16_entry(int H, int Lmax) {
    for (const auto& m : kB16)
        if (m.H == H) return (Lmax <= 16 * m.CG && b16_shape(m, Lmax)) ? &m : nullptr;
    return nullptr;
}

size_t b16_lds(const B16Entry& m) {
    const size_t nrw = 16 * (size_t)m.CG + 1, he = 16 * (size_t)m.NB, nblk = nrw / 16 + 1;
    const size_t kp = (5 * (size_t)m.H + 31) / 32 * 32, ra = 2 * kp + 8, cs = he + 4;
    const size_t sk = 128 / m.CG, skc = m.NB == 1 ? 64 : 0;
    const size_t ebuf = nrw * (he / 2) * 4 + nblk * sk, cbuf = nrw * cs * 4 + nblk * skc;
    const size_t abuf = nrw * ra * 2 + nblk * sk;
    const size_t small = 2 * ebuf + 6 * cbuf;  // exponents, dc f_l, dc f_u, X, Y
    return (small + 15) / 16 * 16 + 2 * abuf;
}

}  // namespace

bool bwd16_supported(int H, int Lmax) { return b16_entry(H, Lmax) != nullptr; }

size_t bwd16_lds(int H, int Lmax) {
    const B16Entry* m = b16_entry(H, Lmax);
    return m ? b16_lds(*m) : 0;
}

hipError_t launch_bwd16(const Dev& D, int H, const float* Ul, const float* Uu, const float* stash,
                        const float* dy_flat, const float* dh_dirs, float* dA, int32_t* done, hipStream_t st) {
    const B16Entry* m = b16_entry(H, D.max_diag);
    if (!m) return hipErrorInvalidValue;
    const B16Shape2* sh = b16_shape(*m, D.max_diag);
    launch(sh->k, dim3(4 * D.n), dim3(64 * (kMatWaves + sh->EW)), b16_lds(*m), st, D, Ul, Uu, stash, dy_flat,
           dh_dirs, dA, done);
    return hipGetLastError();
}

}  // namespace mdl
