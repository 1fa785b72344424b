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
// Each diagonal is done in two phases separated by a barrier.
//  1. Four matrix waves (one per SIMD) take the gate gradients da of the later diagonal s + 1, already in
//     LDS, and form for each of its cells m the products X(m) = da(m) Ul^T and Y(m) = da(m) Uu^T on
//     v_mfma_f32_16x16x32_f16: the parts of dh that m sends to its left and upper predecessors. Then
//     dh(a, b) = dy(a, b) + X(R) + Y(D), and each row of da is read once. Both operands are split
//     into f16 hi + lo pairs (three partial products summed in fp32). Gate gradients have no bound, so
//     each (cell, 16-wide block of hidden units) row of da was scaled by the power of two that brings its
//     largest magnitude into [2^14, 2^15) before it was split; its exponent sits in LDS beside it and the
//     product is scaled back exactly. The K dimension orders da by (hidden unit, gate), the five gates
//     padded to eight.
//  2. All waves do the elementwise part, each thread owning fixed
//     (diagonal position, hidden unit) elements: dc, da, the scale of its
//     row (a maximum over the 16 lanes of a DPP row), the split into the LDS
//     A rows of the next phase 1, and the store of da for the weight
//     gradients. A single wave issues a VALU instruction only every few
//     cycles, so the workgroup is sized to give each thread of the widest
//     diagonal one element (two where the registers do not allow it).
// Rows of the LDS A operand are permuted so the 16 lanes gathering one K
// block read 16 consecutive rows on distinct banks. The forward's gate stash
// and the upstream gradient of each element are prefetched three diagonals
// ahead; the memory states c of the predecessor diagonal come from its own
// prefetch through LDS. The loop is unrolled by four so every step is
// straight code and the compiler's vmcnt waits cover only the prefetch they
// need (loads and stores retire in order on this hardware).
#include "kernels.h"
#include "devmath.h"

#include <type_traits>

namespace mdl {

namespace {

constexpr int kOOB = 0x40000000;  // byte offset past every per-unit range used here (1 GiB)
constexpr int kPD = 3;            // diagonals of prefetch ahead
constexpr int kMatWaves = 4;      // phase 1 on the first four

template <int H>
struct B16Shape {
    static constexpr int NB = (H + 15) / 16;  // blocks of 16 hidden units
    static constexpr int HE = 16 * NB;        // hidden units padded to whole DPP rows
    static constexpr int CG = kMatWaves / NB; // cell groups of the matrix waves
    static constexpr int KA = 128;            // K extent of one successor's da per block: 16 units x 8 slots
    static constexpr int KT = KA / 32;        // K blocks of 32 per (successor, block)
    static_assert(NB <= 2, "hidden size above 32");
};

template <int N>
using IC = std::integral_constant<int, N>;

// exact power-of-two scale 2^E that brings m (> 0) into [2^14, 2^15); 0 for m = 0
__device__ inline int scale_exp(uint32_t mbits) {
    if (mbits == 0) return 0;
    int E = 14 - ((int)((mbits >> 23) & 255) - 127);
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

// f16 pair of a scaled value v (|v| < 2^15): hi is v with its low 13 mantissa bits cleared, which f16
// holds exactly (11 significant bits; below the f16 normal range the rounding is under 2^-25), and
// lo = v - hi rounded to f16, so hi + lo is v to about 2^-21 of |v|
__device__ inline float hi_part(float v) { return __uint_as_float(__float_as_uint(v) & 0xFFFFE000u); }

// NE: elements per thread in phase 2, NT threads: NE NT covers the cells x padded units of the widest diagonal
template <int H, int NE, int NT>
__global__ __launch_bounds__(NT) void k_bwd16(Dev D, const float* __restrict__ Ul, const float* __restrict__ Uu,
                                                    const float* __restrict__ stash,
                                                    const float* __restrict__ dy_flat,
                                                    const float* __restrict__ dh_dirs, float* __restrict__ dA) {
    using Sh = B16Shape<H>;
    constexpr int NB = Sh::NB, HE = Sh::HE, CG = Sh::CG, KA = Sh::KA, KT = Sh::KT;
    constexpr int G = 5 * H;
    const int u = D.units[blockIdx.x];
    const int e = u >> 2, d = u & 3;
    const int y0 = D.rect[4 * e], x0 = D.rect[4 * e + 1], h = D.rect[4 * e + 2], w = D.rect[4 * e + 3];
    const int ry0 = D.real[4 * e], rx0 = D.real[4 * e + 1], rh = D.real[4 * e + 2], rw = D.real[4 * e + 3];
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const bool mat = wave < kMatWaves;
    // phase 1 role of a matrix wave: output block kb, cell group cg; lane (q, col)
    const int kb = (wave % kMatWaves) / CG, cg = (wave % kMatWaves) % CG;
    const int q = lane >> 4, col = lane & 15;

    // Phase 1 forms, for every cell m of the later diagonal s + 1, X(m) = da(m) Ul^T and Y(m) = da(m) Uu^T:
    // the parts of dh that cell m sends to its left and upper predecessors. A wave computes two output
    // column blocks ("pairs") for its 16 cells: with one block of hidden units, X and Y of that block;
    // with two, blocks 0 and 1 of X (kb = 0) or of Y (kb = 1).
    // B operand of pair p: U^T rows in the (unit, gate) K order; for input block bi and K block t the lane
    // holds K rows 32t + 8q + i = 8 (4t + q) + i: unit k' = 16 bi + 4t + q, gate i (zero for i >= 5).
    // Scaled per output column by 2^E and split into f16 hi + lo.
    auto pair_y = [&](int p) { return NB == 1 ? p : kb; };               // pair computes Y (uses Uu)
    auto pair_col = [&](int p) { return 16 * (NB == 1 ? 0 : p) + col; };  // output hidden unit
    f16x8 Bh[2][NB][KT], Bl[2][NB][KT];
    int ec[2];  // the columns' scale exponents, negated
#pragma unroll
    for (int pp = 0; pp < 2; ++pp) {
        float v[NB][KT][8];
        float m = 0.f;
        const float* U = pair_y(pp) ? Uu : Ul;
        const int kc = pair_col(pp);
#pragma unroll
        for (int bi = 0; bi < NB; ++bi)
#pragma unroll
            for (int t = 0; t < KT; ++t)
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const int kp = 16 * bi + 4 * t + q;
                    float x = 0.f;
                    if (mat && kc < H && kp < H && i < 5) x = U[((int64_t)d * H + kc) * G + i * H + kp];
                    v[bi][t][i] = x;
                    m = fmaxf(m, fabsf(x));
                }
        m = fmaxf(m, __shfl_xor(m, 16));
        m = fmaxf(m, __shfl_xor(m, 32));
        const int E = scale_exp(__float_as_uint(m));
        ec[pp] = -E;
#pragma unroll
        for (int bi = 0; bi < NB; ++bi)
#pragma unroll
            for (int t = 0; t < KT; ++t)
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    _Float16 hi, lo;
                    split16(ldexpf(v[bi][t][i], E), hi, lo);
                    Bh[pp][bi][t][i] = hi;
                    Bl[pp][bi][t][i] = lo;
                }
    }

    // LDS, two buffers (later / current diagonal) of NRW rows: the split, scaled da as f16
    // [hi | lo][block][unit][8] (row stride RA halves), the scale exponents [block] (ints), dc*f_l and
    // dc*f_u (row stride CS floats); one buffer each of the phase-1 results X and Y of the later diagonal
    // and of the memory states c of the predecessor diagonal (row stride CS). Diagonal position j lives
    // in row P(j) (below); ZR is a zero row, XR absorbs the writes of idle threads.
    constexpr int RA = 2 * NB * KA + 8, CS = HE + 4;
    constexpr int NRW = 16 * CG + 2, ZR = 16 * CG, XR = 16 * CG + 1;
    constexpr int ABUF = NRW * RA * 2, EBUF = NRW * NB * 4, CBUF = NRW * CS * 4;
    constexpr int OFF_E = 2 * ABUF, OFF_CL = OFF_E + 2 * EBUF, OFF_CU = OFF_CL + 2 * CBUF;
    constexpr int OFF_X = OFF_CU + 2 * CBUF, OFF_Y = OFF_X + CBUF;
    constexpr int OFF_CP = OFF_Y + CBUF;
    constexpr int LDS_BYTES = OFF_CP + CBUF;
    extern __shared__ __align__(16) unsigned char smem[];
    {
        uint32_t* z32 = reinterpret_cast<uint32_t*>(smem);
        for (int i = tid; i < LDS_BYTES / 4; i += NT) z32[i] = 0u;
    }
    const int64_t base = (int64_t)d * D.T + D.cell_off[e];
    const int64_t cells = (int64_t)h * w;
    const int64_t o1 = z1_offset(D.T, H);
    const __amdgpu_buffer_rsrc_t rS4 = rsrc(stash + base * 4 * H, cells * 16 * H);
    const __amdgpu_buffer_rsrc_t rS2 = rsrc(stash + o1 + base * 2 * H, cells * 8 * H);
    const __amdgpu_buffer_rsrc_t rA4 = rsrc(dA + base * 4 * H, cells * 16 * H);
    const __amdgpu_buffer_rsrc_t rA1 = rsrc(dA + o1 + base * H, cells * 4 * H);
    const bool per_dir = dh_dirs != nullptr;
    const __amdgpu_buffer_rsrc_t rU =
        per_dir ? rsrc(dh_dirs + (int64_t)d * D.Hc * D.Wc * H, (int64_t)D.Hc * D.Wc * H * 4)
                : rsrc(dy_flat + D.flat_off[e] * H, (int64_t)rh * rw * H * 4);
    const int S = h + w - 1;

    // Cell j of a diagonal belongs to cell group j % CG and is cell i = j / CG of that group's matrix wave,
    // computed in MFMA row 4(i%4) + i/4; its LDS row P(j) = 16(j % CG) + 4(i%4) + i/4 makes the 16 lanes
    // that gather one K block read 16 consecutive rows. Positions outside [0, 16 CG) map to the zero row.
    auto P = [&](int j) {
        if (j < 0 || j >= 16 * CG) return ZR;
        const int i = j / CG;
        return 16 * (j % CG) + 4 * (i & 3) + (i >> 2);
    };

    // ---- phase 1 constants (matrix waves) ----
    // The lane's A row is its own cell ja = (4 (col & 3) + (col >> 2)) CG + cg of the later diagonal; its
    // output rows r are the cells (4r + q) CG + cg, at LDS rows 16 cg + 4q + r, whose scale exponents the
    // product carries.
    const int oa1 = P((4 * (col & 3) + (col >> 2)) * CG + cg) * RA * 2;
    const int orow = 16 * cg + 4 * q;  // LDS row of output row r: orow + r

    // ---- phase 2 constants: element n of this thread is (position pj, unit pk) ----
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
    int pj[NE], vu[NE], ve[NE];
    bool pk_ok[NE];
    int wa[NE], we[NE], wc[NE];  // own LDS offsets (within a buffer)
    int oc[NE][3];                         // c-row offsets at positions pj - 1, pj, pj + 1
#pragma unroll
    for (int n = 0; n < NE; ++n) {
        const int el = tid + NT * n;
        pj[n] = el / HE;
        const int pk = el - pj[n] * HE, pb = pk / 16, pc = pk - 16 * pb;
        pk_ok[n] = pk < H;
        const int pkc = pk < H ? pk : 0;
        vu[n] = pj[n] * UA + 4 * pkc;
        ve[n] = pj[n] * H + pkc;
        const int pr = P(pj[n]);
        wa[n] = pr * RA * 2 + (pb * KA + 8 * pc) * 2;
        we[n] = (pr * NB + pb) * 4;
        wc[n] = pr * CS * 4 + 4 * pk;
#pragma unroll
        for (int m = 0; m < 3; ++m) oc[n][m] = P(pj[n] + m - 1) * CS * 4 + 4 * pk;
    }
    // writes of elements without a cell go to the discard row, reads of absent successors to the zero row
    const int pk0 = tid % HE, pb0 = pk0 / 16, pc0 = pk0 - 16 * pb0;
    const int xa = XR * RA * 2 + (pb0 * KA + 8 * pc0) * 2, xe = (XR * NB + pb0) * 4, xc = XR * CS * 4 + 4 * pk0;
    const int zc = ZR * CS * 4 + 4 * pk0;

    auto diag_len = [&](int s) {
        if (s < 0 || s >= S) return 0;
        const int lo = s > w - 1 ? s - (w - 1) : 0;
        const int hi = s < h - 1 ? s : h - 1;
        return hi - lo + 1;
    };
    auto diag_lo = [&](int s) { return s > w - 1 ? s - (w - 1) : 0; };

    // forward values of this thread's elements on one diagonal: i, f_l, f_u, o | g, c | dy
    struct Fw {
        f32x4 g4[NE];
        f32x2 g2[NE];
        float dy[NE];
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
            const bool ok = (pj[n] < L1) & pk_ok[n];
            const int el = pe + ve[n];
            f.g4[n] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rS4, ok ? el * 16 : kOOB, 0, 0));
            f.g2[n] = __builtin_bit_cast(f32x2, __builtin_amdgcn_raw_buffer_load_b64(rS2, ok ? el * 8 : kOOB, 0, 0));
            const bool vy = ok & (per_dir | ((pj[n] >= jr0) & (pj[n] < jr1)));
            f.dy[n] = bld(rU, vy ? pu0 + vu[n] : kOOB);
        }
    };

    Fw fs[4];
    // stash index of the first cell of diagonal s and of the prefetch diagonal s - kPD
    int st = (int)cells - 1;  // diagonal S - 1 is the single last cell
    int stz = st;
#pragma unroll
    for (int i = 0; i < kPD; ++i) {
        load_f(S - 1 - i, stz, fs[i]);
        stz -= diag_len(S - 2 - i);
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the loop starts with nothing in flight
    __syncthreads();

    // diagonal s at position POS of the unrolled loop (POS = (S - 1 - s) mod 4): buffer POS & 1 is
    // written, 1 - (POS & 1) holds diagonal s + 1; prefetch set POS is consumed, (POS + kPD) & 3 refilled
    auto step = [&](int s, auto POSc) {
        constexpr int POS = decltype(POSc)::value;
        constexpr int CB = POS & 1;
        const int L = diag_len(s), L1 = diag_len(s + 1);
        // the prefetch: at the top of the step, except in the matrix waves, which issue it inside phase 1 so
        // that its address arithmetic overlaps their LDS reads and products (every wave issues the same memory
        // operations per step)
        const int stz_now = stz;
        stz -= diag_len(s - kPD - 1);
        if (!mat) load_f(s - kPD, stz_now, fs[(POS + kPD) & 3]);
        __builtin_amdgcn_sched_barrier(0);  // keep the prefetch at the top of the step
        const int dn = s >= w - 1 ? 1 : 0;  // successors of position j: right j - dn, down j + 1 - dn
        const unsigned char* ap = smem + (1 - CB) * ABUF;
        const unsigned char* ep = smem + OFF_E + (1 - CB) * EBUF;
        // ---- phase 1: X and Y of the later diagonal, matrix waves only (no global memory inside) ----
        if (mat) {
            // scale exponents of the output rows: read before the products where registers allow
            int er[4][NB];
            auto read_er = [&]() {
#pragma unroll
                for (int r = 0; r < 4; ++r)
#pragma unroll
                    for (int bi = 0; bi < NB; ++bi)
                        er[r][bi] = *reinterpret_cast<const int*>(ep + ((orow + r) * NB + bi) * 4);
            };
            if constexpr (NB == 1) read_er();
            load_f(s - kPD, stz_now, fs[(POS + kPD) & 3]);
            f32x4 acc[2][NB];
#pragma unroll
            for (int pp = 0; pp < 2; ++pp)
#pragma unroll
                for (int bi = 0; bi < NB; ++bi) acc[pp][bi] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int bi = 0; bi < NB; ++bi)
#pragma unroll
                for (int t = 0; t < KT; ++t) {
                    const unsigned char* p = ap + oa1 + (bi * KA + 32 * t + 8 * q) * 2;
                    const f16x8 ah = *reinterpret_cast<const f16x8*>(__builtin_assume_aligned(p, 16));
                    const f16x8 al = *reinterpret_cast<const f16x8*>(__builtin_assume_aligned(p + NB * KA * 2, 16));
#pragma unroll
                    for (int pp = 0; pp < 2; ++pp) {
                        acc[pp][bi] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, Bh[pp][bi][t], acc[pp][bi], 0, 0, 0);
                        acc[pp][bi] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, Bl[pp][bi][t], acc[pp][bi], 0, 0, 0);
                        acc[pp][bi] = __builtin_amdgcn_mfma_f32_16x16x32_f16(al, Bh[pp][bi][t], acc[pp][bi], 0, 0, 0);
                    }
                }
            if constexpr (NB != 1) read_er();
#pragma unroll
            for (int pp = 0; pp < 2; ++pp)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    float v = 0.f;
#pragma unroll
                    for (int bi = 0; bi < NB; ++bi) v += ldexpf(acc[pp][bi][r], ec[pp] - er[r][bi]);
                    *reinterpret_cast<float*>(smem + (pair_y(pp) ? OFF_Y : OFF_X) +
                                              ((orow + r) * CS + pair_col(pp)) * 4) = v;
                }
        }
        // memory states of diagonal s - 1 (prefetched with it) for this diagonal's predecessor terms
#pragma unroll
        for (int n = 0; n < NE; ++n) *reinterpret_cast<float*>(smem + OFF_CP + wc[n]) = fs[(POS + 1) & 3].g2[n][1];
        __syncthreads();
        // ---- phase 2: elementwise, all threads ----
        const Fw& f = fs[POS];
        const unsigned char* clp = smem + OFF_CL + (1 - CB) * CBUF;
        const unsigned char* cup = smem + OFF_CU + (1 - CB) * CBUF;
        unsigned char* aw = smem + CB * ABUF;
        unsigned char* ew = smem + OFF_E + CB * EBUF;
        unsigned char* clw = smem + OFF_CL + CB * CBUF;
        unsigned char* cuw = smem + OFF_CU + CB * CBUF;
        const int pe = st * H;
        // predecessors of position j on diagonal s - 1: left j + dl iff j < Ml, up j + dl - 1 iff j >= 1 - dl
        const int dl = s >= w ? 1 : 0;
        const int lo = diag_lo(s);
        const int Ml = L < s - lo ? L : s - lo;
#pragma unroll
        for (int n = 0; n < NE; ++n) {
            const int j = pj[n];
            const bool ok = (j < L) & pk_ok[n];
            const bool hr = j >= dn, hd = j + 1 - dn < L1;
            const float cl = *reinterpret_cast<const float*>(smem + OFF_CP + (j < Ml ? (dl ? oc[n][2] : oc[n][1]) : zc));
            const float cu = *reinterpret_cast<const float*>(smem + OFF_CP + (j + dl >= 1 ? (dl ? oc[n][1] : oc[n][0]) : zc));
            const int ocr = hr ? (dn ? oc[n][0] : oc[n][1]) : zc;  // right successor's c row, or zero row
            const int ocd = hd ? (dn ? oc[n][1] : oc[n][2]) : zc;  // lower successor's
            // dh: X of the right successor and Y of the lower one (zero rows when absent), plus dy
            const float dh = (*reinterpret_cast<const float*>(smem + OFF_X + ocr) +
                              *reinterpret_cast<const float*>(smem + OFF_Y + ocd)) + f.dy[n];
            const float dcin = *reinterpret_cast<const float*>(clp + ocr) + *reinterpret_cast<const float*>(cup + ocd);
            const float ig = f.g4[n][0], fl = f.g4[n][1], fu = f.g4[n][2], og = f.g4[n][3];
            const float gg = f.g2[n][0], c = f.g2[n][1];
            const float tc = ftanh(c);
            const float dov = dh * tc;
            const float dc = __builtin_fmaf(dh * og, 1.f - tc * tc, dcin);
            const float d0 = dc * gg * ig * (1.f - ig);
            const float d1 = dc * cl * fl * (1.f - fl);
            const float d2 = dc * cu * fu * (1.f - fu);
            const float d3 = dov * og * (1.f - og);
            const float d4 = dc * ig * (1.f - gg * gg);
            // scale of this (cell, block): the largest |da| over the 16 units of the block (non-negative
            // floats order like their bit patterns)
            const float am = fmaxf(fmaxf(fabsf(d0), fabsf(d1)), fmaxf(fmaxf(fabsf(d2), fabsf(d3)), fabsf(d4)));
            const uint32_t mb = row16_max(ok ? __float_as_uint(am) : 0u);
            const int E = scale_exp(mb);
            const float s0 = ldexpf(d0, E), s1 = ldexpf(d1, E), s2 = ldexpf(d2, E), s3 = ldexpf(d3, E),
                        s4 = ldexpf(d4, E);
            const float t0 = hi_part(s0), t1 = hi_part(s1), t2 = hi_part(s2), t3 = hi_part(s3), t4 = hi_part(s4);
            const f16x8 hv = {(_Float16)t0, (_Float16)t1, (_Float16)t2, (_Float16)t3, (_Float16)t4,
                              (_Float16)0, (_Float16)0, (_Float16)0};
            const f16x8 lv = {(_Float16)(s0 - t0), (_Float16)(s1 - t1), (_Float16)(s2 - t2), (_Float16)(s3 - t3),
                              (_Float16)(s4 - t4), (_Float16)0, (_Float16)0, (_Float16)0};
            unsigned char* pa = aw + (ok ? wa[n] : xa);
            *reinterpret_cast<f16x8*>(__builtin_assume_aligned(pa, 16)) = hv;
            *reinterpret_cast<f16x8*>(__builtin_assume_aligned(pa + NB * KA * 2, 16)) = lv;
            *reinterpret_cast<int*>(ew + (ok ? we[n] : xe)) = E;
            *reinterpret_cast<float*>(clw + (ok ? wc[n] : xc)) = dc * fl;
            *reinterpret_cast<float*>(cuw + (ok ? wc[n] : xc)) = dc * fu;
            const int el = pe + ve[n];
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, f32x4{d0, d1, d2, d3}), rA4,
                                                   ok ? el * 16 : kOOB, 0, 0);
            bst(d4, rA1, ok ? el * 4 : kOOB);
        }
        st -= diag_len(s - 1);
        __syncthreads();
    };
    int s = S - 1;
    for (; s - 3 >= 0; s -= 4) {
        step(s, IC<0>{});
        step(s - 1, IC<1>{});
        step(s - 2, IC<2>{});
        step(s - 3, IC<3>{});
    }
    if (s >= 0) step(s, IC<0>{});
    if (s - 1 >= 0) step(s - 1, IC<1>{});
    if (s - 2 >= 0) step(s - 2, IC<2>{});
}

typedef void (*Bwd16Kernel)(Dev, const float*, const float*, const float*, const float*, const float*, float*);

// hidden sizes of the workloads, each with its (elements per thread, threads) shapes in order of preference:
// one element per thread while the widest diagonal fits the workgroup (shorter chains in phase 2), else two
struct B16Shape2 {
    int NE, NT;
    Bwd16Kernel k;
};
struct B16Entry {
    int H, NB, CG;
    B16Shape2 shapes[4];
};
#define MDL_B16S(h, ne, nt) {ne, nt, k_bwd16<h, ne, nt>}
#define MDL_B16(h)                                                                                          \
    {h, B16Shape<h>::NB, B16Shape<h>::CG,                                                                   \
     {MDL_B16S(h, 1, 512), MDL_B16S(h, 1, 640), MDL_B16S(h, 1, 768), MDL_B16S(h, 2, 512)}}
const B16Entry kB16[] = {MDL_B16(16),
                         {32, B16Shape<32>::NB, B16Shape<32>::CG,
                          {MDL_B16S(32, 1, 512), MDL_B16S(32, 2, 512), {0, 0, nullptr}, {0, 0, nullptr}}}};
#undef MDL_B16
#undef MDL_B16S

// the widest diagonal must fit the matrix waves' tiles (16 CG cells) and one of the phase-2 shapes
const B16Shape2* b16_shape(const B16Entry& m, int Lmax) {
    const int elems = Lmax * 16 * m.NB;
    for (const auto& sh : m.shapes)
        if (sh.k && elems <= sh.NE * sh.NT) return &sh;
    return nullptr;
}
const B16Entry* b16_entry(int H, int Lmax) {
    for (const auto& m : kB16)
        if (m.H == H) return (Lmax <= 16 * m.CG && b16_shape(m, Lmax)) ? &m : nullptr;
    return nullptr;
}

size_t b16_lds(const B16Entry& m) {
    const size_t nrw = 16 * (size_t)m.CG + 2, he = 16 * (size_t)m.NB;
    const size_t ra = 2 * (size_t)m.NB * 128 + 8, cs = he + 4;
    return 2 * nrw * ra * 2 + 2 * nrw * m.NB * 4 + 7 * nrw * cs * 4;
}

}  // namespace

bool bwd16_supported(int H, int Lmax) { return b16_entry(H, Lmax) != nullptr; }

size_t bwd16_lds(int H, int Lmax) {
    const B16Entry* m = b16_entry(H, Lmax);
    return m ? b16_lds(*m) : 0;
}

hipError_t launch_bwd16(const Dev& D, int H, const float* Ul, const float* Uu, const float* stash,
                        const float* dy_flat, const float* dh_dirs, float* dA, hipStream_t st) {
    const B16Entry* m = b16_entry(H, D.max_diag);
    if (!m) return hipErrorInvalidValue;
    const B16Shape2* sh = b16_shape(*m, D.max_diag);
    launch(sh->k, dim3(4 * D.n), dim3(sh->NT), b16_lds(*m), st, D, Ul, Uu, stash, dy_flat, dh_dirs, dA);
    return hipGetLastError();
}

}  // namespace mdl
