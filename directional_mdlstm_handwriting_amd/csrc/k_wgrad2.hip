// k_wgrad2.hip — weight and input gradients after the reverse wavefront, software-pipelined.
//
// The same sums as k_wgrad.hip (RETURNN §4.2: after the recurrent part is
// back-propagated, the gradients of the weights and inputs are matrix products
// over the whole batch):
//     [dWx; db; dUl; dUu][d] = sum over computed cells p of r(p)^T da_d(p),
//     r(p) = [x(p), 1, h_left(p), h_up(p)],       dx(p) = sum over d of da_d(p) Wx[d]^T,
// for shapes fixed at compile time. One workgroup takes one group of the
// layout's weight-gradient split (a few cell ranges of about the same total
// size for every workgroup, so all compute units finish together) for all
// four directions, WPD waves per direction, and walks it in tiles of TP = 32 cells. The global loads of tile t+1 (16-byte
// loads of the predecessors' h and of the gate gradients in their [cell][k][4] layout)
// are issued before tile t is computed from LDS, so their latency hides
// behind the matrix-core work. Each thread stages a fixed share of one cell
// of each tile and works out that cell's pixel, predecessors and stash
// position itself, so the loads wait on no shared table. The tile sits in
// LDS component-major: one row of TP cells for each component of r and each
// gate column of da.
// r^T da runs on v_mfma_f32_16x16x32_bf16 (K = the tile's 32 cells) where a
// wave's tiles leave the registers for it: every fp32 operand is split exactly
// into three bf16 pieces, v = v1 + v2 + v3 (each piece the leading 8
// significant bits of what is left; bf16 keeps fp32's exponent range, so
// nothing is scaled), and the product keeps the six terms v_i w_j with
// i + j <= 4 (the dropped ones are below 2^-23 of v w), accumulated in fp32
// smallest first. Otherwise it runs on v_mfma_f32_16x16x4_f32 (fp32 products
// and sums, K = 4 cells per instruction). Each wave owns all M tiles of its
// direction and a share of its N tiles. dx runs on v_mfma_f32_4x4x1f32, whose 16 independent
// 4 x 4 blocks fit the few input channels without padding (the 16 x 16
// instruction would waste three quarters of its columns at C = 4): every wave
// takes a share of the gate-gradient columns of all four directions, the
// directions are added across lanes, and the waves' shares in a fixed order.
// LDS row strides are chosen so the fragment reads of a wave hit distinct banks.
// The workgroups' partials are reduced in workgroup order by k_wgrad_reduce (k_wgrad.hip).
#include "kernels.h"
#include "devmath.h"

namespace mdl {

namespace {

constexpr int kOOBw = 0x7ffffff0;  // byte offset past every buffer range: loads return 0

template <int C, int H>
struct WgShape {
    static constexpr int G = 5 * H, R = C + 1 + 2 * H;
    static constexpr int TP = 32;                         // cells per tile: the K extent of one product
    static constexpr int MT = (R + 15) / 16, NT = (G + 15) / 16;
    static constexpr int WPD = (MT * NT + 31) / 32;       // waves per direction: at most 32 tiles per wave
    static constexpr int NTW = (NT + WPD - 1) / WPD;      // N tiles per wave (bound)
    static constexpr int RR = 16 * MT, NR = 16 * NT;      // LDS rows of r components and of gate columns
    // the product on bf16 pieces where a wave's split fragments fit its registers beside its accumulators
    // (at most 16 tiles per wave), else on fp32 v_mfma_f32_16x16x4_f32
    static constexpr bool BF = MT * NTW <= 16;
    // LDS row stride: 16-byte rows (4 mod 32 floats) for the 8-cell fragment reads of the bf16 product,
    // 2 (mod 32) for the single-cell reads of the fp32 one, so either read pattern hits distinct banks
    static constexpr int TPD = BF ? TP + 4 : TP + 2;
    static constexpr int VH = H % 4 == 0 ? 4 : (H % 2 == 0 ? 2 : 1);    // h / dA1 load width
    static constexpr int NTH = 64 * WPD;                  // threads per direction
    static constexpr int TPC = NTH / TP;                  // threads per cell of a tile in the loads
    static constexpr int NVH = 2 * H / VH, NV1 = H / VH;  // h and dA1 vectors of a cell
    static constexpr int NHL = (NVH + TPC - 1) / TPC;     // h loads per thread
    static constexpr int ND4 = (H + TPC - 1) / TPC;       // dA4 loads per thread (16 bytes)
    static constexpr int ND1 = (NV1 + TPC - 1) / TPC;     // dA1 loads per thread
    static constexpr int NXL = (C + TPC - 1) / TPC;       // x loads per thread
    static constexpr int NWV = 4 * WPD;                   // waves of the workgroup
    static constexpr int NPW = (G + NWV - 1) / NWV;       // da columns of the dx product per wave
    static constexpr int NC4 = (C + 3) / 4;               // groups of 4 input channels
    static constexpr int LATE = 0;                        // next tile's loads after the products (registers)
    static_assert(C <= 16, "dx product assumes at most 16 input channels");
    static_assert(NWV * NPW <= NR, "dx column shares stay inside the gate-column rows");
    static_assert(NTH % TP == 0 && (TPC & (TPC - 1)) == 0, "whole power-of-two thread groups per cell");
};

template <int N>
struct VecOf;
template <>
struct VecOf<1> { typedef float T; };
template <>
struct VecOf<2> { typedef f32x2 T; };
template <>
struct VecOf<4> { typedef f32x4 T; };

template <int VB>
__device__ inline typename VecOf<VB>::T vload(__amdgpu_buffer_rsrc_t r, int off) {
    if constexpr (VB == 4) return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
    else if constexpr (VB == 2) return __builtin_bit_cast(f32x2, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
    else return bld(r, off);
}
template <int VB>
__device__ inline float vget(const typename VecOf<VB>::T& v, int i) {
    if constexpr (VB == 1) return v;
    else return v[i];
}

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// the exact split v = v1 + v2 + v3 of eight fp32 values into three bf16 pieces, each piece the leading 8
// significant bits (sign, exponent and 7 mantissa bits: the upper half of the fp32 pattern) of what the
// pieces before it leave; the last remainder has at most 8 significant bits and is exact in bf16.
// Pairs of values pack into one register as (low half: even value, high half: odd value).
__device__ inline void split3(const f32x4& x0, const f32x4& x1, u32x4 (&p)[3]) {
    uint32_t u[3][8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const float v = i < 4 ? x0[i] : x1[i - 4];
        const uint32_t b0 = __float_as_uint(v);
        const float e1 = v - __uint_as_float(b0 & 0xFFFF0000u);
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

// position of region-local cell (ly, lx) of an h x w region in direction d's diagonal-major order
__device__ inline int stash_pos(int h, int w, int ly, int lx, int d) {
    const int a = (d & 2) ? h - 1 - ly : ly;
    const int b = (d & 1) ? w - 1 - lx : lx;
    const int s = a + b;
    return (int)dg_start(h, w, s) + (a - dg_lo(h, w, s));
}

// One workgroup's group grp: its partial sums and the input gradient of its cells.
template <bool BF16, int C, int H>
__device__ __forceinline__ void wgrad_group(const Dev& D, const void* __restrict__ xc, const float* __restrict__ hdirs,
                                            const float* __restrict__ dA, const float* __restrict__ Wx,
                                            float* __restrict__ part, float* __restrict__ dx_flat,
                                            float* __restrict__ dx_canvas, const int grp) {
    using S = WgShape<C, H>;
    constexpr int G = S::G, R = S::R, MT = S::MT, NT = S::NT, WPD = S::WPD, NTW = S::NTW, TP = S::TP;
    constexpr int RR = S::RR, NR = S::NR, TPD = S::TPD, VH = S::VH, NTH = S::NTH, NWV = S::NWV, NPW = S::NPW,
                  NC4 = S::NC4;
    constexpr int TPC = S::TPC, NVH = S::NVH, NV1 = S::NV1, NHL = S::NHL, ND4 = S::ND4, ND1 = S::ND1, NXL = S::NXL;
    constexpr int LATE_LOADS = S::LATE;
    constexpr bool BF = S::BF;
    constexpr int XB = BF16 ? 2 : 4;
    typedef typename VecOf<VH>::T HV;
    const int sg0 = D.groups[grp], nsg = D.groups[grp + 1] - sg0;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: per-wave descriptors
    const int d = wave / WPD, sub = wave % WPD;  // direction, share of its N tiles
    const int td = tid - d * NTH;                // thread index within the direction
    const int i16 = lane & 15, q = lane >> 4;
    const int nt0 = sub * NTW;
    const int64_t plane = (int64_t)D.Hc * D.Wc * H;

    // this workgroup's segments, read once into LDS (a global load inside the loop would wait on the
    // stores): region y0, x0, h, w; real pixels y0, x0, h, w; stash and flat offsets; cell range
    __shared__ int sgt[kGroupSegs][12];
    if (tid < nsg) {
        const int sg = sg0 + tid, e = D.segs[3 * sg];
        int* o = sgt[tid];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            o[i] = D.rect[4 * e + i];
            o[4 + i] = D.real[4 * e + i];
        }
        o[8] = (int)D.cell_off[e];
        o[9] = (int)D.flat_off[e];
        o[10] = D.segs[3 * sg + 1];
        o[11] = D.segs[3 * sg + 2];
    }

    // LDS: r [4][RR][TPD] (component m of r, then the tile's cells), gate gradients [4][NR][TPD] (gate
    // column n = g H + k), dx shares of the waves [NWV][TP][C], and two slots of the tile's cell table
    // (pixel, flat index) for the dx store; rows past R and G stay zero
    extern __shared__ __align__(16) unsigned char smem[];
    float* rs = reinterpret_cast<float*>(smem);
    float* das = rs + 4 * RR * TPD;
    float* dxs = das + 4 * NR * TPD;
    int* tpix = reinterpret_cast<int*>(dxs + NWV * TP * C);  // [2][TP]
    int* tflat = tpix + 2 * TP;                              // [2][TP]
    constexpr int NWORDS = 4 * RR * TPD + 4 * NR * TPD + NWV * TP * C + 4 * TP;
    for (int i = tid; i < NWORDS; i += blockDim.x) reinterpret_cast<uint32_t*>(smem)[i] = 0u;
    __syncthreads();
    for (int i = tid; i < 4 * TP; i += blockDim.x) rs[((i / TP) * RR + C) * TPD + i % TP] = 1.f;  // the bias row
    int ntiles = 0;
    for (int sg = 0; sg < nsg; ++sg) ntiles += (sgt[sg][11] - sgt[sg][10] + TP - 1) / TP;

    // loads: thread td of a direction stages cell lc = td / TPC of each tile, vectors pt, pt + TPC, ...
    const int lc = td / TPC, pt = td % TPC;

    // this wave's direction: its h plane and its gate gradients, each one 32-bit range
    const __amdgpu_buffer_rsrc_t rH = rsrc(hdirs + d * plane, plane * 4);
    const __amdgpu_buffer_rsrc_t rA4 = rsrc(dA + (int64_t)d * D.T * 4 * H, (int64_t)D.T * 16 * H);
    const __amdgpu_buffer_rsrc_t rA1 = rsrc(dA + z1_offset(D.T, H) + (int64_t)d * D.T * H, (int64_t)D.T * 4 * H);
    const __amdgpu_buffer_rsrc_t rX = rsrc(xc, (int64_t)D.Hc * D.Wc * C * XB);

    // staged values of one tile for this thread's direction
    HV vh[NHL];
    f32x4 vd4[ND4];
    HV vd1[ND1];
    float vx[NXL];
    auto issue_loads = [&](int sg, int lt, int slot) {
        // this thread's cell (tile lt of segment sg): canvas pixel, predecessors in direction d, position
        // in d's stash order
        const int* S = sgt[sg];
        const int y0 = S[0], x0 = S[1], h = S[2], w = S[3];
        const int cell0 = S[8];
        const int qc = S[10] + lt * TP + lc;
        const bool ok = qc < S[11];
        const int ly = qc / w, lx = qc - ly * w;
        const int pix = ok ? (y0 + ly) * D.Wc + x0 + lx : -1;
        const bool lok = ok & ((d & 1) ? lx < w - 1 : lx > 0);  // left predecessor (y, x - sx)
        const bool uok = ok & ((d & 2) ? ly < h - 1 : ly > 0);  // upper predecessor (y - sy, x)
        const int srcl = pix + ((d & 1) ? 1 : -1), srcu = pix + ((d & 2) ? D.Wc : -D.Wc);
        const int cst = ok ? stash_pos(h, w, ly, lx, d) : 0;
        if (d == 0 && pt == 0) {  // the dx store's table
            const int qy = y0 + ly - S[4], qx = x0 + lx - S[5];
            tpix[slot * TP + lc] = pix;
            tflat[slot * TP + lc] = (ok & (qy < S[6]) & (qx < S[7])) ? S[9] + qy * S[7] + qx : -1;
        }
#pragma unroll
        for (int i = 0; i < NHL; ++i) {
            const int v = pt + i * TPC;  // vector of [2][H / VH]: left then upper predecessor
            const bool up = v >= NV1;
            const int kv = up ? v - NV1 : v;
            const bool pok = (v < NVH) & (up ? uok : lok);
            vh[i] = vload<VH>(rH, pok ? ((up ? srcu : srcl) * H + kv * VH) * 4 : kOOBw);
        }
#pragma unroll
        for (int i = 0; i < ND4; ++i) {
            const int k = pt + i * TPC;
            vd4[i] = vload<4>(rA4, ((k < H) & ok) ? ((cell0 + cst) * H + k) * 16 : kOOBw);
        }
#pragma unroll
        for (int i = 0; i < ND1; ++i) {
            const int kv = pt + i * TPC;
            vd1[i] = vload<VH>(rA1, ((kv < NV1) & ok) ? ((cell0 + cst) * H + kv * VH) * 4 : kOOBw);
        }
#pragma unroll
        for (int i = 0; i < NXL; ++i) {
            const int k = pt + i * TPC;
            const int off = ((k < C) & ok) ? (pix * C + k) * XB : kOOBw;
            if constexpr (BF16) vx[i] = __uint_as_float((uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rX, off, 0, 0) << 16);
            else vx[i] = bld(rX, off);
        }
    };
    auto write_lds = [&]() {
        float* rsd = rs + d * RR * TPD + lc;
        float* dad = das + d * NR * TPD + lc;
#pragma unroll
        for (int i = 0; i < NHL; ++i) {
            const int v = pt + i * TPC;
            if (v < NVH) {
                const int up = v >= NV1 ? 1 : 0, kv = v - up * NV1;
#pragma unroll
                for (int j = 0; j < VH; ++j) rsd[(C + 1 + up * H + kv * VH + j) * TPD] = vget<VH>(vh[i], j);
            }
        }
#pragma unroll
        for (int i = 0; i < ND4; ++i) {
            const int k = pt + i * TPC;
            if (k < H) {
#pragma unroll
                for (int g = 0; g < 4; ++g) dad[(g * H + k) * TPD] = vd4[i][g];
            }
        }
#pragma unroll
        for (int i = 0; i < ND1; ++i) {
            const int kv = pt + i * TPC;
            if (kv < NV1) {
#pragma unroll
                for (int j = 0; j < VH; ++j) dad[(4 * H + kv * VH + j) * TPD] = vget<VH>(vd1[i], j);
            }
        }
#pragma unroll
        for (int i = 0; i < NXL; ++i) {
            const int k = pt + i * TPC;
            if (k < C) rsd[k * TPD] = vx[i];
        }
    };

    // dx = sum over d of da_d Wx_d^T on v_mfma_f32_4x4x1f32 (16 blocks of 4 x 4 x 1): block b = lane / 4
    // holds cell group b % 4 (4 cells) of direction b / 4 against 4 input channels, so every lane does
    // useful work with C <= 4 and the direction sum is two cross-lane additions. Each wave takes NPW
    // consecutive gate columns (same for all four directions); its Wx_d values stay in registers.
    const int xd = lane >> 4, xi = lane & 3, xcell = lane & 15;  // block direction; row / channel in block; cell
    const int col0 = wave * NPW;
    float wxr[NC4][NPW];
#pragma unroll
    for (int g4 = 0; g4 < NC4; ++g4)
#pragma unroll
        for (int sc = 0; sc < NPW; ++sc) {
            const int col = col0 + sc, ch = 4 * g4 + xi;
            wxr[g4][sc] = (col < G && ch < C) ? Wx[((int64_t)xd * C + ch) * G + col] : 0.f;
        }
    const bool want_dx = dx_flat != nullptr || dx_canvas != nullptr;

    f32x4 acc[MT][NTW];
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int j = 0; j < NTW; ++j) acc[m][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    int sg = 0, lt = 0;  // the tile being computed: segment, tile within it
    issue_loads(0, 0, 0);
    for (int t = 0; t < ntiles; ++t) {
        const int slot = t & 1;
        int sgn = sg, ltn = lt + 1;  // the next tile
        if (ltn * TP >= sgt[sg][11] - sgt[sg][10]) {
            ++sgn;
            ltn = 0;
        }
        write_lds();
        __syncthreads();
        // the next tile's loads go out once the products no longer need their registers; they are in flight
        // through the dx part and the barrier (at hidden sizes whose product leaves room, right away)
        if (LATE_LOADS == 0 && t + 1 < ntiles) issue_loads(sgn, ltn, (t + 1) & 1);
        if constexpr (BF) {
            // A fragment of M tile m: component 16 m + i16 of r over the cells 8q .. 8q + 7; B fragment of N tile
            // j: gate column 16 (nt0 + j) + i16 over the same cells; both split into three bf16 pieces
            const float* rsd = rs + (d * RR + i16) * TPD + 8 * q;
            const float* dad = das + (d * NR + 16 * nt0 + i16) * TPD + 8 * q;
            u32x4 ap[MT][3];
#pragma unroll
            for (int m = 0; m < MT; ++m)
                split3(*reinterpret_cast<const f32x4*>(rsd + 16 * m * TPD),
                       *reinterpret_cast<const f32x4*>(rsd + 16 * m * TPD + 4), ap[m]);
#pragma unroll
            for (int j = 0; j < NTW; ++j) {
                if (nt0 + j < NT) {
                    u32x4 bp[3];
                    split3(*reinterpret_cast<const f32x4*>(dad + 16 * j * TPD),
                           *reinterpret_cast<const f32x4*>(dad + 16 * j * TPD + 4), bp);
#pragma unroll
                    for (int m = 0; m < MT; ++m) {
                        f32x4 a = acc[m][j];
                        // the six terms of order <= 2^-16, smallest first
                        a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, ap[m][2]),
                                                                    __builtin_bit_cast(bf16x8, bp[0]), a, 0, 0, 0);
                        a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, ap[m][1]),
                                                                    __builtin_bit_cast(bf16x8, bp[1]), a, 0, 0, 0);
                        a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, ap[m][0]),
                                                                    __builtin_bit_cast(bf16x8, bp[2]), a, 0, 0, 0);
                        a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, ap[m][1]),
                                                                    __builtin_bit_cast(bf16x8, bp[0]), a, 0, 0, 0);
                        a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, ap[m][0]),
                                                                    __builtin_bit_cast(bf16x8, bp[1]), a, 0, 0, 0);
                        a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, ap[m][0]),
                                                                    __builtin_bit_cast(bf16x8, bp[0]), a, 0, 0, 0);
                        acc[m][j] = a;
                    }
                }
            }
        } else {
            // K step ks: cell 4 ks + q of the tile; A component 16 m + i16, B gate column 16 (nt0 + j) + i16
            const float* rsd = rs + (d * RR + i16) * TPD + q;
            const float* dad = das + (d * NR + 16 * nt0 + i16) * TPD + q;
#pragma unroll
            for (int ks = 0; ks < TP / 4; ++ks) {
                float af[MT], bf[NTW];
#pragma unroll
                for (int m = 0; m < MT; ++m) af[m] = rsd[16 * m * TPD + 4 * ks];
#pragma unroll
                for (int j = 0; j < NTW; ++j) bf[j] = nt0 + j < NT ? dad[16 * j * TPD + 4 * ks] : 0.f;
#pragma unroll
                for (int m = 0; m < MT; ++m)
#pragma unroll
                    for (int j = 0; j < NTW; ++j)
                        if (nt0 + j < NT)
                            acc[m][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(af[m], bf[j], acc[m][j], 0, 0, 0);
            }
        }
        if (LATE_LOADS != 0 && t + 1 < ntiles) issue_loads(sgn, ltn, (t + 1) & 1);
        // this wave's share of dx for the tile's cells, 16 cells at a time
        if (want_dx) {
#pragma unroll
            for (int m2 = 0; m2 < TP / 16; ++m2) {
                const float* arow = das + (xd * NR + col0) * TPD + 16 * m2 + xcell;
                f32x4 dacc[NC4];
#pragma unroll
                for (int g4 = 0; g4 < NC4; ++g4) dacc[g4] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int sc = 0; sc < NPW; ++sc) {
                    const float av = arow[sc * TPD];  // gate columns from G on are zero rows
#pragma unroll
                    for (int g4 = 0; g4 < NC4; ++g4)
                        dacc[g4] = __builtin_amdgcn_mfma_f32_4x4x1f32(av, wxr[g4][sc], dacc[g4], 0, 0, 0);
                }
#pragma unroll
                for (int g4 = 0; g4 < NC4; ++g4)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        // lanes l, l^16, l^32, l^48 hold the four directions of one (cell, channel);
                        // every lane ends with the same sum (fp addition commutes)
                        float v = dacc[g4][r];
                        v += __shfl_xor(v, 16);
                        v += __shfl_xor(v, 32);
                        const int ch = 4 * g4 + xi;
                        if (lane < 16 && ch < C) dxs[(wave * TP + 16 * m2 + 4 * (xcell >> 2) + r) * C + ch] = v;
                    }
            }
        }
        __syncthreads();
        {
            const int* pix = tpix + slot * TP;
            const int* flat = tflat + slot * TP;
            for (int o = tid; o < TP * C; o += blockDim.x) {
                const int c = o / C, chn = o - c * C;
                if (pix[c] < 0) continue;
                float v = dxs[c * C + chn];
#pragma unroll
                for (int wv = 1; wv < NWV; ++wv) v += dxs[(wv * TP + c) * C + chn];  // waves in order
                if (dx_flat && flat[c] >= 0) dx_flat[(int64_t)flat[c] * C + chn] = v;
                if (dx_canvas) dx_canvas[(int64_t)pix[c] * C + chn] = flat[c] >= 0 ? v : 0.f;
            }
        }
        sg = sgn;
        lt = ltn;
    }
    // partial sums of this workgroup: part[group][d][R][G]
    float* out = part + ((int64_t)grp * 4 + d) * R * G;
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int j = 0; j < NTW; ++j) {
            const int col = 16 * (nt0 + j) + i16;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = 16 * m + 4 * q + r;
                if (nt0 + j < NT && row < R && col < G) out[(int64_t)row * G + col] = acc[m][j][r];
            }
        }
}

// one workgroup per group; groups whose processed flag is set (done by the overlapping launch) are skipped
template <bool BF16, int C, int H>
__global__ __launch_bounds__((256 * WgShape<C, H>::WPD)) void k_wgrad2(Dev D, const void* __restrict__ xc,
                                                                      const float* __restrict__ hdirs,
                                                                      const float* __restrict__ dA,
                                                                      const float* __restrict__ Wx,
                                                                      float* __restrict__ part,
                                                                      float* __restrict__ dx_flat,
                                                                      float* __restrict__ dx_canvas,
                                                                      const int32_t* __restrict__ processed) {
    const int grp = blockIdx.x;
    if (processed != nullptr && processed[grp] != 0) return;
    wgrad_group<BF16, C, H>(D, xc, hdirs, dA, Wx, part, dx_flat, dx_canvas, grp);
}

// Thread 0 of an overlapping workgroup claims the next group in readiness order and waits until every
// reverse-wavefront unit of its examples has finished. The counters are polled without ordering (no cache
// invalidation per poll); one acquire fence once they are all complete orders the group's reads after the
// units' stores. Each wait is bounded by `budget` shader-clock cycles; a group not ready by then is left to
// the launch that follows the reverse wavefront, and the stop flag ends all claiming. Returns the group, or -1.
__device__ int claim_ready_group(const Dev& D, const OverlapFlags& F, long long budget) {
    if (__hip_atomic_load(F.stop, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0) return -1;
    const int qi = __hip_atomic_fetch_add(F.queue, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (qi >= D.ngroups) return -1;
    const int g = D.gorder[qi];
    const unsigned long long t0 = __builtin_amdgcn_s_memtime();
    for (int sg = D.groups[g]; sg < D.groups[g + 1]; ++sg) {
        const int e = D.segs[3 * sg];
        while (__hip_atomic_load(F.done + e, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < 4) {
            if ((long long)(__builtin_amdgcn_s_memtime() - t0) > budget) {
                __hip_atomic_store(F.stop, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                return -1;
            }
            __builtin_amdgcn_s_sleep(16);
        }
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    return g;
}

// The weight gradient beside the reverse wavefront: a few persistent workgroups (on the compute units the
// wavefront leaves free) take the groups in the order their examples finish, each after that example's
// four units have signalled; every group they complete is marked processed.
template <bool BF16, int C, int H>
__global__ __launch_bounds__((256 * WgShape<C, H>::WPD)) void k_wgrad2_overlap(Dev D, const void* __restrict__ xc,
                                                                              const float* __restrict__ hdirs,
                                                                              const float* __restrict__ dA,
                                                                              const float* __restrict__ Wx,
                                                                              float* __restrict__ part,
                                                                              float* __restrict__ dx_flat,
                                                                              float* __restrict__ dx_canvas,
                                                                              OverlapFlags F, long long budget) {
    __shared__ int s_grp;
    // Thread 0's work of an iteration (mark the group finished last, claim the next) is one region between
    // barriers. Two separate thread-0 regions, one at the end of an iteration and one at the start of the
    // next, may be merged across the loop's back edge by the compiler into a path on which thread 0 leaves
    // the loop body while the rest of its wave goes on to the next barrier without it.
    int prev = -1;  // the group this workgroup finished last (the same in every thread)
    for (;;) {
        if (threadIdx.x == 0) {
            if (prev >= 0) __hip_atomic_store(F.processed + prev, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
            s_grp = claim_ready_group(D, F, budget);
        }
        __syncthreads();
        const int g = s_grp;
        __syncthreads();
        if (g < 0) break;
        wgrad_group<BF16, C, H>(D, xc, hdirs, dA, Wx, part, dx_flat, dx_canvas, g);
        __threadfence();  // the group's partial sums and dx before its processed flag
        __syncthreads();
        prev = g;
    }
}

template <bool BF16, int C, int H>
size_t wg2_lds() {
    using S = WgShape<C, H>;
    constexpr size_t TP = S::TP;
    return 4 * (4 * (size_t)S::RR * S::TPD + 4 * (size_t)S::NR * S::TPD + (size_t)S::NWV * TP * C + 4 * TP);
}

typedef void (*Wg2Kernel)(Dev, const void*, const float*, const float*, const float*, float*, float*, float*,
                          const int32_t*);
typedef void (*Wg2OverlapKernel)(Dev, const void*, const float*, const float*, const float*, float*, float*, float*,
                                 OverlapFlags, long long);

struct Wg2Entry {
    bool bf16;
    int C, H, threads;
    size_t lds;
    Wg2Kernel k;
    Wg2OverlapKernel ko;
};
#define MDL_WG2(bf, c, h) \
    {bf, c, h, 256 * WgShape<c, h>::WPD, wg2_lds<bf, c, h>(), k_wgrad2<bf, c, h>, k_wgrad2_overlap<bf, c, h>}
const Wg2Entry* wg2_entry(int C, int H, bool bf16) {
    static const Wg2Entry table[] = {MDL_WG2(false, 4, 16), MDL_WG2(true, 4, 16), MDL_WG2(false, 4, 32),
                                     MDL_WG2(true, 4, 32),  MDL_WG2(false, 4, 2), MDL_WG2(false, 6, 10),
                                     MDL_WG2(false, 1, 4)};
    for (const auto& m : table)
        if (m.C == C && m.H == H && m.bf16 == bf16) return &m;
    return nullptr;
}
#undef MDL_WG2

}  // namespace

bool wgrad2_supported(int C, int H, int dtype) { return wg2_entry(C, H, dtype != 0) != nullptr; }

size_t wgrad2_lds_bytes(int C, int H, int dtype) {
    const Wg2Entry* m = wg2_entry(C, H, dtype != 0);
    return m ? m->lds : 0;
}

hipError_t launch_wgrad2(const Dev& D, const void* x_canvas, int dtype, int C, int H, const float* h_dirs,
                         const float* dA, const float* Wx, float* part, float* dx_flat, float* dx_canvas,
                         const int32_t* processed, hipStream_t st) {
    const Wg2Entry* m = wg2_entry(C, H, dtype != 0);
    if (!m) return hipErrorInvalidValue;
    launch(m->k, dim3((unsigned)D.ngroups), dim3(m->threads), m->lds, st, D, x_canvas, h_dirs, dA, Wx,
           part, dx_flat, dx_canvas, processed);
    return hipGetLastError();
}

hipError_t launch_wgrad2_overlap(const Dev& D, const void* x_canvas, int dtype, int C, int H, const float* h_dirs,
                                 const float* dA, const float* Wx, float* part, float* dx_flat, float* dx_canvas,
                                 const OverlapFlags& F, int workgroups, long long budget, hipStream_t st) {
    const Wg2Entry* m = wg2_entry(C, H, dtype != 0);
    if (!m || workgroups < 1) return hipErrorInvalidValue;
    launch(m->ko, dim3((unsigned)workgroups), dim3(m->threads), m->lds, st, D, x_canvas, h_dirs, dA, Wx, part,
           dx_flat, dx_canvas, F, budget);
    return hipGetLastError();
}

}  // namespace mdl
