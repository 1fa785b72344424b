// k_wgrad2.hip — weight and input gradients after the reverse wavefront, software-pipelined.
//
// The same sums as k_wgrad.hip (RETURNN §4.2: after the recurrent part is
// back-propagated, the gradients of the weights and inputs are matrix products
// over the whole batch):
//     [dWx; db; dUl; dUu][d] = sum over computed cells p of r(p)^T da_d(p),
//     r(p) = [x(p), 1, h_left(p), h_up(p)],       dx(p) = sum over d of da_d(p) Wx[d]^T,
// for shapes fixed at compile time. A task is one direction of one group of the
// layout's weight-gradient split (a few cell ranges of about the same total size
// for every group); a workgroup of NWV waves takes one task at a time and walks
// it in tiles of TP = 64 cells. The global loads of tile t+1 (16-byte loads of
// the predecessors' h and of the gate gradients in their [cell][k][4] layout)
// are issued before tile t is computed from LDS, so their latency hides behind
// the matrix-core work. Each thread stages a fixed share of one cell of each
// tile and works out that cell's pixel, predecessors and stash position itself,
// so the loads wait on no shared table. The tile sits in LDS component-major:
// one row of TP cells for each component of r and each gate column of da.
// r^T da runs on v_mfma_f32_16x16x32_bf16 (K = 32 cells, two steps a tile): every fp32
// operand is split exactly into three bf16 pieces, v = v1 + v2 + v3 (each piece
// the leading 8 significant bits of what is left; bf16 keeps fp32's exponent
// range, so nothing is scaled), and the product keeps the six terms v_i w_j with
// i + j <= 4 (the dropped ones are below 2^-23 of v w), accumulated in fp32
// smallest first. Each wave owns all M tiles of the direction and a share of its
// N tiles, at most 16 tiles in all, so the split fragments fit its registers
// beside the accumulators. The direction's share of dx runs on
// v_mfma_f32_4x4x1f32, whose 16 independent 4 x 4 blocks fit the few input
// channels without padding: every wave takes a share of the gate-gradient
// columns, a quarter of them in each group of 16 lanes, the quarters are added
// across lanes and the waves' shares in a fixed order; the four directions'
// shares are added, in direction order, by k_dx_sum. The task partial sums are
// reduced in group order by k_wgrad_reduce (k_wgrad.hip). LDS row strides are
// chosen so the fragment reads of a wave hit distinct banks.
#include "kernels.h"
#include "devmath.h"

namespace mdl {

namespace {

constexpr int kOOBw = 0x7ffffff0;  // byte offset past every buffer range: loads return 0

// waves of a workgroup: 4 (2 when there are fewer than 4 N tiles), or 8 where 4 would leave a wave more than
// 16 product tiles
constexpr int wg_waves(int MT, int NT) {
    return NT < 4 ? 2 : (MT * ((NT + 3) / 4) <= 16 ? 4 : 8);
}

template <int C, int H>
struct WgShape {
    static constexpr int G = 5 * H, R = C + 1 + 2 * H;
    static constexpr int TP = 64;                         // cells per tile: two K = 32 product steps
    static constexpr int MT = (R + 15) / 16, NT = (G + 15) / 16;
    static constexpr int NWV = wg_waves(MT, NT);          // waves of the workgroup, all on the task's direction
    static constexpr int NTW = (NT + NWV - 1) / NWV;      // N tiles per wave (bound)
    static constexpr int NR = 16 * NT;                    // LDS rows of gate columns
    static constexpr int TPD = TP + 4;                    // gate-column row stride (floats): 4 mod 32 dwords
    static constexpr int TPD16 = TP + 8;                  // r-piece row stride (bf16 values): 4 mod 32 dwords
    static constexpr int RPS = (R + 1) * TPD16;           // r-piece plane: R rows and one zero row
    static constexpr int RPB = (3 * RPS * 2 + 15) / 16 * 16;  // bytes of the three r-piece planes
    static constexpr int VH = H % 4 == 0 ? 4 : (H % 2 == 0 ? 2 : 1);    // h / dA1 load width
    static constexpr int NTH = 64 * NWV;                  // threads of the workgroup
    static constexpr int TPC = NTH / TP;                  // threads per cell of a tile in the loads
    static constexpr int NVH = 2 * H / VH, NV1 = H / VH;  // h and dA1 vectors of a cell
    static constexpr int NHL = (NVH + TPC - 1) / TPC;     // h loads per thread
    static constexpr int ND4 = (H + TPC - 1) / TPC;       // dA4 loads per thread (16 bytes)
    static constexpr int ND1 = (NV1 + TPC - 1) / TPC;     // dA1 loads per thread
    static constexpr int NXL = (C + TPC - 1) / TPC;       // x loads per thread
    static constexpr int NPW = (G + 4 * NWV - 1) / (4 * NWV) * 4;  // dx gate columns per wave
    static constexpr int CP = (C + 3) / 4 * 4;            // dx weight row: channels padded to 16-byte vectors
    static constexpr int NWX = NWV * NPW;                 // dx weight rows (gate columns, zero from G on)
    // workgroups per compute unit the registers are held to (the LDS of two fits at every shape used)
    static constexpr int OCC = 2;
    // tiles whose loads are in flight ahead of the one computed: two where a second set of staging registers
    // leaves the occupancy as it is (hidden sizes up to 16), else one
    static constexpr int PF = H <= 16 ? 2 : 1;
    static_assert(MT * NTW <= 16, "at most 16 product tiles per wave");
    static_assert(C <= 16, "dx accumulators: at most 16 input channels");
    static_assert(TP == 64, "dx: one cell of the tile per lane");
    static_assert(NWV * NPW <= NR, "dx column shares stay inside the gate-column rows");
    static_assert(NTH % TP == 0 && (TPC & (TPC - 1)) == 0, "whole power-of-two thread groups per cell");
};

template <int N>
struct IC {
    static constexpr int value = N;
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

// rows of a band in the weight-gradient walk (a power of two)
constexpr int kBand = 8;

// j / dv for 0 <= j < 2^22 and dv >= 1, from the hardware reciprocal of dv (within one ulp: the estimate is
// off by at most one)
__device__ inline int qdiv(int j, int dv) {
    const int q = (int)((float)j * __builtin_amdgcn_rcpf((float)dv));
    const int r = j - q * dv;
    return q + (r >= dv ? 1 : 0) - (r < 0 ? 1 : 0);
}

// position of region-local cell (ly, lx) of an h x w region in direction d's diagonal-major order
__device__ inline int stash_pos(int h, int w, int ly, int lx, int d) {
    const int a = (d & 2) ? h - 1 - ly : ly;
    const int b = (d & 1) ? w - 1 - lx : lx;
    const int s = a + b;
    return (int)dg_start(h, w, s) + (a - dg_lo(h, w, s));
}

// One task: direction d of group grp. Its partial sums go to part[grp][d], its share of dx (the tile
// cells' da_d Wx[d]^T, if dx is wanted) to dxp[d][cell] (cells numbered as in the layout's cell
// offsets, row-major inside each region).
template <bool BF16, int C, int H>
__device__ __forceinline__ void wgrad_task(const Dev& D, const void* __restrict__ xc, const float* __restrict__ hdirs,
                                           const float* __restrict__ dA, const float* __restrict__ Wx,
                                           float* __restrict__ part, float* __restrict__ dxp, const int task) {
    using S = WgShape<C, H>;
    constexpr int G = S::G, R = S::R, MT = S::MT, NT = S::NT, NTW = S::NTW, TP = S::TP;
    constexpr int NR = S::NR, TPD = S::TPD, TPD16 = S::TPD16, RPS = S::RPS, VH = S::VH, NWV = S::NWV,
                  NPW = S::NPW;
    constexpr int TPC = S::TPC, NVH = S::NVH, NV1 = S::NV1, NHL = S::NHL, ND4 = S::ND4, ND1 = S::ND1, NXL = S::NXL;
    // the launch's block size as a compile-time stride: the block size read at run time is a memory load, and
    // its wait would also wait for every tile load in flight
    constexpr int NTH = S::NTH;
    constexpr int XB = BF16 ? 2 : 4, PF = S::PF;
    typedef typename VecOf<VH>::T HV;
    const int grp = task >> 2, d = task & 3;
    const int sg0 = D.groups[grp], nsg = D.groups[grp + 1] - sg0;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: per-wave descriptors
    const int i16 = lane & 15, q = lane >> 4;
    const int nt0 = wave * NTW;
    const int64_t plane = (int64_t)D.Hc * D.Wc * H;

    // this task's segments, read once into LDS (a global load inside the loop would wait on the
    // stores): region y0, x0, h, w; real pixels y0, x0, h, w; stash and flat offsets; cell range; its walk
    // order. A segment (a row-major cell range of the region) is walked as its head (the rest of a row
    // it starts inside, in row order), its body (the whole rows after it, in bands of kBand rows, each
    // band column after column) and its tail (the start of the row it ends inside, in row order): inside
    // a band a cell's upper predecessor is the cell before it and its left predecessor kBand cells back,
    // so both are loaded while the cell that loaded them first is recent (still in the L2), and a load
    // instruction still covers runs of kBand neighbouring pixels of a row. Fields 12..16: head cells, first
    // body row, body rows, head row, head column. (Two workgroups of the largest shape fill the compute
    // unit's LDS but for about 1.5 KB, which holds this table and the cell indices below.)
    __shared__ int sgt[kGroupSegs][17];
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
        const int first = D.segs[3 * sg + 1], end = D.segs[3 * sg + 2], w = o[3];
        const int ya = first / w, xa = first - ya * w, ye = end / w;
        o[10] = first;
        o[11] = end;
        o[12] = ya == ye ? end - first : (xa > 0 ? w - xa : 0);
        o[13] = ya + (xa > 0 ? 1 : 0);
        o[14] = ya == ye ? 0 : ye - o[13];
        o[15] = ya;
        o[16] = xa;
    }
    // region-local row-major index of each cell of the tile, for the dx store (written after the tile's
    // first barrier, read after its second)
    __shared__ int cids[TP];

    // LDS: r as its three bf16 pieces [3][R + 1][TPD16] (component m of r, then the tile's cells; row R stays
    // zero and stands for the rows of the last M tile past R), written split by the thread that loads the value,
    // so each value is split once; gate gradients [NR][TPD] in fp32 (gate column n = g H + k; rows past G stay
    // zero), split by the one wave whose N tile holds them; dx shares of the waves [NWV][TP][C]
    extern __shared__ __align__(16) unsigned char smem[];
    uint16_t* rp = reinterpret_cast<uint16_t*>(smem);
    float* das = reinterpret_cast<float*>(smem + S::RPB);
    float* dxs = das + NR * TPD;
    float* wxs = dxs + NWV * TP * C;  // Wx_d^T [NWX][CP]: row = gate column, read by every lane at once
    constexpr int NWORDS = S::RPB / 4 + NR * TPD + NWV * TP * C + S::NWX * S::CP;
    for (int i = tid; i < NWORDS; i += NTH) reinterpret_cast<uint32_t*>(smem)[i] = 0u;
    __syncthreads();
    for (int i = tid; i < TP; i += NTH) rp[C * TPD16 + i] = 0x3F80;  // the bias row: 1 = 1 + 0 + 0
    for (int i = tid; i < G * C; i += NTH) {
        const int col = i / C, c = i - col * C;
        wxs[col * S::CP + c] = Wx[((int64_t)d * C + c) * G + col];
    }
    int ntiles = 0;
    for (int sg = 0; sg < nsg; ++sg) ntiles += (sgt[sg][11] - sgt[sg][10] + TP - 1) / TP;

    // loads: thread tid stages cell lc = tid / TPC of each tile, vectors pt, pt + TPC, ...
    const int lc = tid / TPC, pt = tid % TPC;

    // the direction's h plane and gate gradients, each one 32-bit range
    const __amdgpu_buffer_rsrc_t rH = rsrc(hdirs + d * plane, plane * 4);
    const __amdgpu_buffer_rsrc_t rA4 = rsrc(dA + (int64_t)d * D.T * 4 * H, (int64_t)D.T * 16 * H);
    const __amdgpu_buffer_rsrc_t rA1 = rsrc(dA + z1_offset(D.T, H) + (int64_t)d * D.T * H, (int64_t)D.T * 4 * H);
    const __amdgpu_buffer_rsrc_t rX = rsrc(xc, (int64_t)D.Hc * D.Wc * C * XB);

    // staged values of one tile for this thread (x as its stored bits: converting it here would wait for the load)
    HV vh[PF][NHL];
    f32x4 vd4[PF][ND4];
    HV vd1[PF][ND1];
    uint32_t vx[PF][NXL];
    int vci[PF];  // region-local row-major index of the staged cell
    auto issue_loads = [&](auto Bc, int sg, int lt) {
        constexpr int B = decltype(Bc)::value;
        // this thread's cell (tile lt of segment sg): canvas pixel, predecessors in direction d, position
        // in d's stash order
        const int* Sg = sgt[sg];
        const int y0 = Sg[0], x0 = Sg[1], h = Sg[2], w = Sg[3];
        const int cell0 = Sg[8];
        const int wi = lt * TP + lc;  // position in the segment's walk
        const bool ok = wi < Sg[11] - Sg[10];
        const int nhead = Sg[12], yb0 = Sg[13], nrows = Sg[14], nbody = nrows * w;
        int ly, lx;
        if (wi < nhead) {
            ly = Sg[15];
            lx = Sg[16] + wi;
        } else if (wi < nhead + nbody) {
            const int j = wi - nhead;
            const int nfull = nrows / kBand, fullc = nfull * kBand * w;
            if (j < fullc) {
                const int b = qdiv(j, kBand * w);
                const int jj = j - b * kBand * w;
                lx = jj / kBand;
                ly = yb0 + b * kBand + (jj - lx * kBand);
            } else {
                const int rbl = nrows - nfull * kBand, jj = j - fullc;
                lx = qdiv(jj, rbl);
                ly = yb0 + nfull * kBand + (jj - lx * rbl);
            }
        } else {
            ly = yb0 + nrows;
            lx = wi - nhead - nbody;
        }
        vci[B] = ly * w + lx;
        const int pix = ok ? (y0 + ly) * D.Wc + x0 + lx : -1;
        const bool lok = ok & ((d & 1) ? lx < w - 1 : lx > 0);  // left predecessor (y, x - sx)
        const bool uok = ok & ((d & 2) ? ly < h - 1 : ly > 0);  // upper predecessor (y - sy, x)
        const int srcl = pix + ((d & 1) ? 1 : -1), srcu = pix + ((d & 2) ? D.Wc : -D.Wc);
        const int cst = ok ? stash_pos(h, w, ly, lx, d) : 0;
#pragma unroll
        for (int i = 0; i < NHL; ++i) {
            const int v = pt + i * TPC;  // vector of [2][H / VH]: left then upper predecessor
            const bool up = v >= NV1;
            const int kv = up ? v - NV1 : v;
            const bool pok = (v < NVH) & (up ? uok : lok);
            vh[B][i] = vload<VH>(rH, pok ? ((up ? srcu : srcl) * H + kv * VH) * 4 : kOOBw);
        }
#pragma unroll
        for (int i = 0; i < ND4; ++i) {
            const int k = pt + i * TPC;
            vd4[B][i] = vload<4>(rA4, ((k < H) & ok) ? ((cell0 + cst) * H + k) * 16 : kOOBw);
        }
#pragma unroll
        for (int i = 0; i < ND1; ++i) {
            const int kv = pt + i * TPC;
            vd1[B][i] = vload<VH>(rA1, ((kv < NV1) & ok) ? ((cell0 + cst) * H + kv * VH) * 4 : kOOBw);
        }
#pragma unroll
        for (int i = 0; i < NXL; ++i) {
            const int k = pt + i * TPC;
            const int off = ((k < C) & ok) ? (pix * C + k) * XB : kOOBw;
            if constexpr (BF16) vx[B][i] = __builtin_amdgcn_raw_buffer_load_b16(rX, off, 0, 0);
            else vx[B][i] = __builtin_amdgcn_raw_buffer_load_b32(rX, off, 0, 0);
        }
    };
    // component `row` of r for this thread's cell, as three bf16 pieces: each the upper half of what the
    // pieces before it leave (v = v1 + v2 + v3 exactly)
    auto put_r = [&](int row, float v) {
        uint16_t* o = rp + row * TPD16 + lc;
        const uint32_t b0 = __float_as_uint(v);
        const float e1 = v - __uint_as_float(b0 & 0xFFFF0000u);
        const uint32_t b1 = __float_as_uint(e1);
        const float e2 = e1 - __uint_as_float(b1 & 0xFFFF0000u);
        o[0] = (uint16_t)(b0 >> 16);
        o[RPS] = (uint16_t)(b1 >> 16);
        o[2 * RPS] = (uint16_t)(__float_as_uint(e2) >> 16);
    };
    auto write_lds = [&](auto Bc) {
        constexpr int B = decltype(Bc)::value;
        float* dad = das + lc;
#pragma unroll
        for (int i = 0; i < NHL; ++i) {
            const int v = pt + i * TPC;
            if (v < NVH) {
                const int up = v >= NV1 ? 1 : 0, kv = v - up * NV1;
#pragma unroll
                for (int j = 0; j < VH; ++j) put_r(C + 1 + up * H + kv * VH + j, vget<VH>(vh[B][i], j));
            }
        }
#pragma unroll
        for (int i = 0; i < ND4; ++i) {
            const int k = pt + i * TPC;
            if (k < H) {
#pragma unroll
                for (int g = 0; g < 4; ++g) dad[(g * H + k) * TPD] = vd4[B][i][g];
            }
        }
#pragma unroll
        for (int i = 0; i < ND1; ++i) {
            const int kv = pt + i * TPC;
            if (kv < NV1) {
#pragma unroll
                for (int j = 0; j < VH; ++j) dad[(4 * H + kv * VH + j) * TPD] = vget<VH>(vd1[B][i], j);
            }
        }
#pragma unroll
        for (int i = 0; i < NXL; ++i) {
            const int k = pt + i * TPC;
            if (k < C) put_r(k, __uint_as_float(BF16 ? vx[B][i] << 16 : vx[B][i]));
        }
    };

    // dx_d = da_d Wx_d^T: each wave takes NPW consecutive gate columns (col0 on), each lane one cell of the
    // tile, with fp32 multiply-adds in column order; a column's weights are one LDS read that every lane
    // shares (columns from G on are zeros, in both operands)
    const int col0 = wave * NPW;
    const bool want_dx = dxp != nullptr;

    f32x4 acc[MT][NTW];
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int j = 0; j < NTW; ++j) acc[m][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    // tile order: the segments' tiles one after another
    auto advance = [&](int& sgv, int& ltv) {
        if ((ltv + 1) * TP >= sgt[sgv][11] - sgt[sgv][10]) {
            ++sgv;
            ltv = 0;
        } else {
            ++ltv;
        }
    };
    int sg = 0, lt = 0;    // the tile being computed: segment, tile within it
    int sgl = 0, ltl = 0;  // the last tile whose loads were issued
    issue_loads(IC<0>{}, 0, 0);
    if constexpr (PF == 2)
        if (ntiles > 1) {
            advance(sgl, ltl);
            issue_loads(IC<1>{}, sgl, ltl);
        }
    // tile t, staged in buffer t % PF
    auto tile = [&](int t, auto Bc) {
        write_lds(Bc);
        __syncthreads();
        // every wave has stored the tile before: its cells' indices, before the next loads reuse vci
        if (want_dx && pt == 0) cids[lc] = vci[decltype(Bc)::value];
        // the loads of tile t + PF go out once tile t is in LDS, into the buffer it leaves; they are in flight
        // through the products, the dx part and the barrier (with PF = 2, also through all of tile t + 1)
        if (t + PF < ntiles) {
            advance(sgl, ltl);
            issue_loads(Bc, sgl, ltl);
        }
#pragma unroll
        for (int kh = 0; kh < TP / 32; ++kh) {
            // K step kh: cells 32 kh .. 32 kh + 31 of the tile. A fragment of M tile m: component 16 m + i16 of r
            // (the zero row from R on) over the cells 32 kh + 8q .. + 7, its three pieces read from LDS; B
            // fragment of N tile j: gate column 16 (nt0 + j) + i16 over the same cells, split here. The B pieces
            // of the wave's N tiles stay in registers while the M tiles' A pieces are read in turn.
            const float* dad = das + i16 * TPD + 32 * kh + 8 * q;
            // a wave with fewer than NTW N tiles repeats its last one in the spare slots (products not stored),
            // so the product sequence has no branches
            u32x4 bp[NTW][3];
#pragma unroll
            for (int j = 0; j < NTW; ++j) {
                const int nj = min(nt0 + j, NT - 1);
                split3(*reinterpret_cast<const f32x4*>(dad + 16 * nj * TPD),
                       *reinterpret_cast<const f32x4*>(dad + 16 * nj * TPD + 4), bp[j]);
            }
            // A pieces of M tile m + 1 are read while the products of tile m run
            auto read_a = [&](int m, u32x4 (&ap)[3]) {
                const uint16_t* ar = rp + min(16 * m + i16, R) * TPD16 + 32 * kh + 8 * q;
#pragma unroll
                for (int k = 0; k < 3; ++k)
                    ap[k] = *reinterpret_cast<const u32x4*>(__builtin_assume_aligned(ar + k * RPS, 16));
            };
            u32x4 apb[2][3];
            read_a(0, apb[0]);
#pragma unroll
            for (int m = 0; m < MT; ++m) {
                if (m + 1 < MT) read_a(m + 1, apb[(m + 1) & 1]);
                const u32x4 (&ap)[3] = apb[m & 1];
                // term a_ia b_ib of every N tile of the wave (independent accumulators back to back)
                auto term = [&](int ia, int ib) {
#pragma unroll
                    for (int j = 0; j < NTW; ++j)
                        acc[m][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            __builtin_bit_cast(bf16x8, ap[ia]), __builtin_bit_cast(bf16x8, bp[j][ib]), acc[m][j], 0,
                            0, 0);
                };
                // the six terms of order <= 2^-16, smallest first
                term(2, 0);
                term(1, 1);
                term(0, 2);
                term(1, 0);
                term(0, 1);
                term(0, 0);
            }
        }
        // this wave's share of dx_d for the tile's cells
        if (want_dx) {
            const float* arow = das + col0 * TPD + lane;
            const float* wrow = wxs + col0 * S::CP;
            float dv[C];
#pragma unroll
            for (int c = 0; c < C; ++c) dv[c] = 0.f;
#pragma unroll
            for (int i = 0; i < NPW; ++i) {
                const float a = arow[i * TPD];
#pragma unroll
                for (int c4 = 0; c4 < S::CP / 4; ++c4) {
                    const f32x4 wv = *reinterpret_cast<const f32x4*>(wrow + i * S::CP + 4 * c4);
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        if (4 * c4 + j < C) dv[4 * c4 + j] = __builtin_fmaf(a, wv[j], dv[4 * c4 + j]);
                }
            }
#pragma unroll
            for (int c = 0; c < C; ++c) dxs[(wave * TP + lane) * C + c] = dv[c];
        }
        __syncthreads();
        if (want_dx) {
            // each cell's C values at its place in the cell numbering (row-major inside the region)
            const int* Sg = sgt[sg];
            const int nc = min(TP, Sg[11] - Sg[10] - lt * TP);
            float* out = dxp + ((int64_t)d * D.T + Sg[8]) * C;
            const int* ci = cids;
            for (int o = tid; o < nc * C; o += NTH) {
                float v = dxs[o];
#pragma unroll
                for (int wv = 1; wv < NWV; ++wv) v += dxs[wv * TP * C + o];  // waves in order
                const int c = o / C;
                out[(int64_t)ci[c] * C + (o - c * C)] = v;
            }
        }
        advance(sg, lt);
    };
    for (int t = 0; t < ntiles; t += PF) {
        tile(t, IC<0>{});
        if constexpr (PF == 2)
            if (t + 1 < ntiles) tile(t + 1, IC<1>{});
    }
    // partial sums of this task: part[group][d][R][G]
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

// one workgroup per task (direction-minor: task = 4 group + direction)
template <bool BF16, int C, int H>
__global__ __launch_bounds__((64 * WgShape<C, H>::NWV), (WgShape<C, H>::OCC)) void k_wgrad2(Dev D, const void* __restrict__ xc,
                                                                     const float* __restrict__ hdirs,
                                                                     const float* __restrict__ dA,
                                                                     const float* __restrict__ Wx,
                                                                     float* __restrict__ part,
                                                                     float* __restrict__ dxp) {
    wgrad_task<BF16, C, H>(D, xc, hdirs, dA, Wx, part, dxp, blockIdx.x);
}

// Thread 0 of a workgroup beside the reverse wavefront takes its next task: the next queue position
// (unless the stop flag is set) whose taken flag it is first to set (the launch after the wavefront sets
// them too), then waits until the reverse-wavefront unit of the task's direction has finished on every
// example of the group: the flags are polled without ordering (no cache invalidation per poll) and one
// acquire fence, once they are all set, orders the task's reads after the units' stores. Each wait is
// bounded by `budget` shader-clock cycles; a task not ready by then goes on the abandoned list (done after
// both launches) and the stop flag ends claiming beside the wavefront. For the abandoned list, the next
// entry. Returns the task, or -1 once there is none to take.
__device__ int claim_task(const Dev& D, const OverlapFlags& F, int mode, long long budget) {
    if (mode == kClaimAbandoned) {
        const int i = __hip_atomic_fetch_add(F.abq, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        return i < __hip_atomic_load(F.nab, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ? F.abandoned[i] : -1;
    }
    int qi;
    do {
        if (__hip_atomic_load(F.stop, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0) return -1;
        qi = __hip_atomic_fetch_add(F.queue, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (qi >= 4 * D.ngroups) return -1;
    } while (__hip_atomic_exchange(F.taken + qi, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0);
    const int task = D.gorder[qi];
    const int g = task >> 2, d = task & 3;
    const unsigned long long t0 = __builtin_amdgcn_s_memtime();
    for (int sg = D.groups[g]; sg < D.groups[g + 1]; ++sg) {
        const int u = 4 * D.segs[3 * sg] + d;
        while (__hip_atomic_load(F.done + u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 0) {
            if ((long long)(__builtin_amdgcn_s_memtime() - t0) > budget) {
                const int k = __hip_atomic_fetch_add(F.nab, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                F.abandoned[k] = task;
                __hip_atomic_store(F.stop, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                return -1;
            }
            __builtin_amdgcn_s_sleep(16);
        }
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    return task;
}

// Tasks claimed one after another until none is left, beside the reverse wavefront (a few persistent
// workgroups on the compute units it leaves free, taking the tasks in the order their units finish) or,
// after both launches, from the abandoned list.
template <bool BF16, int C, int H>
__global__ __launch_bounds__((64 * WgShape<C, H>::NWV), (WgShape<C, H>::OCC)) void k_wgrad2_claim(Dev D, const void* __restrict__ xc,
                                                                           const float* __restrict__ hdirs,
                                                                           const float* __restrict__ dA,
                                                                           const float* __restrict__ Wx,
                                                                           float* __restrict__ part,
                                                                           float* __restrict__ dxp,
                                                                           OverlapFlags F, int mode,
                                                                           long long budget) {
    __shared__ int s_task;
    // Thread 0's claim is the only thread-0 region of an iteration, and barriers close every iteration:
    // the compiler may otherwise merge thread-0 regions across the loop's back edge into a path on which
    // thread 0 leaves the loop body while the rest of its wave goes on to the next barrier without it.
    for (;;) {
        if (threadIdx.x == 0) s_task = claim_task(D, F, mode, budget);
        __syncthreads();
        const int task = s_task;
        __syncthreads();
        if (task < 0) break;
        wgrad_task<BF16, C, H>(D, xc, hdirs, dA, Wx, part, dxp, task);
        __syncthreads();
    }
}

// After the reverse wavefront on its stream: workgroup b takes queue position b unless a workgroup beside
// the wavefront has taken it (every unit is complete, so nothing is waited for).
template <bool BF16, int C, int H>
__global__ __launch_bounds__((64 * WgShape<C, H>::NWV), (WgShape<C, H>::OCC)) void k_wgrad2_drain(Dev D, const void* __restrict__ xc,
                                                                           const float* __restrict__ hdirs,
                                                                           const float* __restrict__ dA,
                                                                           const float* __restrict__ Wx,
                                                                           float* __restrict__ part,
                                                                           float* __restrict__ dxp,
                                                                           OverlapFlags F) {
    __shared__ int s_taken;
    const int qi = blockIdx.x;
    if (threadIdx.x == 0)
        s_taken = __hip_atomic_exchange(F.taken + qi, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    if (s_taken != 0) return;
    wgrad_task<BF16, C, H>(D, xc, hdirs, dA, Wx, part, dxp, D.gorder[qi]);
}

// dx(p) = ((dx_0(p) + dx_1(p)) + dx_2(p)) + dx_3(p) over the computed cells of example blockIdx.y: dx_flat at
// the real pixels, dx_canvas at every computed cell (zero outside the real pixels)
__global__ __launch_bounds__(256) void k_dx_sum(Dev D, int C, const float* __restrict__ dxp,
                                                float* __restrict__ dx_flat, float* __restrict__ dx_canvas) {
    const int e = blockIdx.y;
    const int y0 = D.rect[4 * e], x0 = D.rect[4 * e + 1], w = D.rect[4 * e + 3];
    const int ry0 = D.real[4 * e], rx0 = D.real[4 * e + 1], rh = D.real[4 * e + 2], rw = D.real[4 * e + 3];
    const int64_t n = (int64_t)D.rect[4 * e + 2] * w * C;
    const int64_t base = D.cell_off[e] * C, TC = D.T * C;
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t cell = i / C;
        const int ch = (int)(i - cell * C);
        const int ly = (int)(cell / w), lx = (int)(cell - (int64_t)ly * w);
        const float* p = dxp + base + i;
        const float v = ((p[0] + p[TC]) + p[2 * TC]) + p[3 * TC];
        const int y = y0 + ly, x = x0 + lx;
        const bool real = (y >= ry0) & (y < ry0 + rh) & (x >= rx0) & (x < rx0 + rw);
        if (dx_canvas) dx_canvas[((int64_t)y * D.Wc + x) * C + ch] = real ? v : 0.f;
        if (dx_flat && real) dx_flat[(D.flat_off[e] + (int64_t)(y - ry0) * rw + (x - rx0)) * C + ch] = v;
    }
}

template <bool BF16, int C, int H>
size_t wg2_lds() {
    using S = WgShape<C, H>;
    return (size_t)S::RPB + 4 * ((size_t)S::NR * S::TPD + (size_t)S::NWV * S::TP * C + (size_t)S::NWX * S::CP);
}

typedef void (*Wg2Kernel)(Dev, const void*, const float*, const float*, const float*, float*, float*);
typedef void (*Wg2ClaimKernel)(Dev, const void*, const float*, const float*, const float*, float*, float*,
                               OverlapFlags, int, long long);
typedef void (*Wg2DrainKernel)(Dev, const void*, const float*, const float*, const float*, float*, float*,
                               OverlapFlags);

struct Wg2Entry {
    bool bf16;
    int C, H, threads;
    size_t lds;
    Wg2Kernel k;
    Wg2ClaimKernel kc;
    Wg2DrainKernel kd;
};
#define MDL_WG2(bf, c, h) \
    {bf, c, h, 64 * WgShape<c, h>::NWV, wg2_lds<bf, c, h>(), k_wgrad2<bf, c, h>, k_wgrad2_claim<bf, c, h>, \
     k_wgrad2_drain<bf, c, h>}
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
                         const float* dA, const float* Wx, float* part, float* dxp, hipStream_t st) {
    const Wg2Entry* m = wg2_entry(C, H, dtype != 0);
    if (!m) return hipErrorInvalidValue;
    launch(m->k, dim3(4u * (unsigned)D.ngroups), dim3(m->threads), m->lds, st, D, x_canvas, h_dirs, dA, Wx, part,
           dxp);
    return hipGetLastError();
}

hipError_t launch_wgrad2_claim(const Dev& D, const void* x_canvas, int dtype, int C, int H, const float* h_dirs,
                               const float* dA, const float* Wx, float* part, float* dxp, const OverlapFlags& F,
                               WgClaim mode, int workgroups, long long budget, size_t lds_hold, hipStream_t st) {
    const Wg2Entry* m = wg2_entry(C, H, dtype != 0);
    if (!m || budget < 0) return hipErrorInvalidValue;
    if (mode == kClaimDrain)
        launch(m->kd, dim3(4u * (unsigned)D.ngroups), dim3(m->threads), m->lds, st, D, x_canvas, h_dirs, dA, Wx, part,
               dxp, F);
    else if (workgroups < 1)
        return hipErrorInvalidValue;
    else
        launch(m->kc, dim3((unsigned)workgroups), dim3(m->threads),
               mode == kClaimBeside ? std::max(m->lds, lds_hold) : m->lds, st, D, x_canvas, h_dirs, dA, Wx, part,
               dxp, F, (int)mode, budget);
    return hipGetLastError();
}

hipError_t launch_dx_sum(const Dev& D, int C, const float* dxp, float* dx_flat, float* dx_canvas, hipStream_t st) {
    if (!dx_flat && !dx_canvas) return hipSuccess;
    launch(k_dx_sum, dim3(64, (unsigned)D.n), dim3(256), 0, st, D, C, dxp, dx_flat, dx_canvas);
    return hipGetLastError();
}

}  // namespace mdl
