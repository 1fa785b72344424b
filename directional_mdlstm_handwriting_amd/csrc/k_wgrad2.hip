// k_wgrad2.hip — weight and input gradients after the reverse wavefront, software-pipelined.
//
// The same sums as k_wgrad.hip (RETURNN §4.2: after the recurrent part is
// back-propagated, the gradients of the weights and inputs are matrix products
// over the whole batch):
//     [dWx; db; dUl; dUu][d] = sum over computed cells p of r(p)^T da_d(p),
//     r(p) = [x(p), 1, h_left(p), h_up(p)],       dx(p) = sum over d of da_d(p) Wx[d]^T,
// for shapes fixed at compile time. One workgroup takes one row chunk of an
// example for all four directions, WPD waves per direction, and walks it in
// tiles of TP cells. The global loads of tile t+1 (16-byte loads of the
// predecessors' h and of the gate gradients in their [cell][k][4] layout)
// are issued before tile t is computed from LDS, so their latency hides
// behind the matrix-core work; the chunk's cell table (pixel, flat index,
// stash index per direction, predecessor flags) is built one tile ahead.
// r^T da runs on v_mfma_f32_16x16x4_f32 (fp32 products and sums, K = 4
// cells per instruction); each wave owns all M tiles of its direction and a
// share of its N tiles. dx runs on the same instruction (A = da, B = Wx^T in
// registers), and the four directions' dx are added in a fixed order. LDS row
// strides are chosen so the fragment reads of a wave hit distinct banks.
// Chunk partials are reduced in chunk order by k_wgrad_reduce (k_wgrad.hip).
#include "kernels.h"
#include "devmath.h"

namespace mdl {

namespace {

constexpr int kOOBw = 0x7ffffff0;  // byte offset past every buffer range: loads return 0
constexpr int TP = 32;             // cells per tile (8 K steps)

template <int C, int H>
struct WgShape {
    static constexpr int G = 5 * H, R = C + 1 + 2 * H;
    static constexpr int MT = (R + 15) / 16, NT = (G + 15) / 16;
    static constexpr int WPD = (MT * NT + 15) / 16;       // waves per direction: at most 16 tiles per wave
    static constexpr int NTW = (NT + WPD - 1) / WPD;      // N tiles per wave (bound)
    static constexpr int RP = MT % 2 ? 16 * MT : 16 * MT + 16;  // r row stride: 16 (mod 32) floats
    static constexpr int DS = G + 1 + ((4 - G % 4) % 4);  // da row stride: 1 (mod 4), > G (column G stays 0)
    static constexpr int VH = H % 4 == 0 ? 4 : (H % 2 == 0 ? 2 : 1);    // h / dA1 load width
    static constexpr int NTH = 64 * WPD;                  // threads per direction
    static constexpr int NHL = (TP * 2 * H / VH + NTH - 1) / NTH;   // h loads per thread
    static constexpr int ND4 = (TP * H + NTH - 1) / NTH;            // dA4 loads per thread (16 bytes)
    static constexpr int ND1 = (TP * H / VH + NTH - 1) / NTH;       // dA1 loads per thread
    static constexpr int NXL = (TP * C + NTH - 1) / NTH;            // x loads per thread
    static constexpr int KX = (G + 3) / 4;                // K steps of the dx product
    static_assert(C <= 16, "dx product assumes at most 16 input channels");
    static_assert(DS % 4 == 1 && DS > G, "da row stride");
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

// position of region-local cell (ly, lx) of an h x w region in direction d's diagonal-major order
__device__ inline int stash_pos(int h, int w, int ly, int lx, int d) {
    const int a = (d & 2) ? h - 1 - ly : ly;
    const int b = (d & 1) ? w - 1 - lx : lx;
    const int s = a + b;
    return (int)dg_start(h, w, s) + (a - dg_lo(h, w, s));
}

template <bool BF16, int C, int H>
__global__ __launch_bounds__((256 * WgShape<C, H>::WPD)) void k_wgrad2(Dev D, const void* __restrict__ xc,
                                                                      const float* __restrict__ hdirs,
                                                                      const float* __restrict__ dA,
                                                                      const float* __restrict__ Wx,
                                                                      float* __restrict__ part,
                                                                      float* __restrict__ dx_flat,
                                                                      float* __restrict__ dx_canvas) {
    using S = WgShape<C, H>;
    constexpr int G = S::G, R = S::R, MT = S::MT, NT = S::NT, WPD = S::WPD, NTW = S::NTW;
    constexpr int RP = S::RP, DS = S::DS, VH = S::VH, NTH = S::NTH, KX = S::KX;
    constexpr int XB = BF16 ? 2 : 4;
    typedef typename VecOf<VH>::T HV;
    const int ch = blockIdx.x;
    const int e = D.chunks[3 * ch], r0 = D.chunks[3 * ch + 1], r1 = D.chunks[3 * ch + 2];
    const int y0 = D.rect[4 * e], x0 = D.rect[4 * e + 1], h = D.rect[4 * e + 2], w = D.rect[4 * e + 3];
    const int ry0 = D.real[4 * e], rx0 = D.real[4 * e + 1], rh = D.real[4 * e + 2], rw = D.real[4 * e + 3];
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: per-wave descriptors
    const int d = wave / WPD, sub = wave % WPD;  // direction, share of its N tiles
    const int td = tid - d * NTH;                // thread index within the direction
    const int i16 = lane & 15, q = lane >> 4;
    const int nt0 = sub * NTW;
    const int ncell = (r1 - r0) * w;
    const int ntiles = (ncell + TP - 1) / TP;
    const int cell0 = (int)D.cell_off[e];
    const int64_t plane = (int64_t)D.Hc * D.Wc * H;

    // LDS: r rows [4][TP][RP], gate gradients [4][TP][DS] (units k: gates 0..3 at 4k + g, gate 4 at 4H + k),
    // per-direction dx [4][TP][C], cell tables [3][TP] of pix, flat, flags and the four stash positions
    extern __shared__ __align__(16) unsigned char smem[];
    float* rs = reinterpret_cast<float*>(smem);
    float* das = rs + 4 * TP * RP;
    float* dxs = das + 4 * TP * DS;
    int* tpix = reinterpret_cast<int*>(dxs + 4 * TP * C);
    int* tflat = tpix + 3 * TP;
    int* tflag = tflat + 3 * TP;
    int* tcst = tflag + 3 * TP;  // [3][4][TP]
    constexpr int NWORDS = 4 * TP * RP + 4 * TP * DS + 4 * TP * C + 3 * TP * 7;
    for (int i = tid; i < NWORDS; i += blockDim.x) reinterpret_cast<uint32_t*>(smem)[i] = 0u;
    __syncthreads();
    for (int i = tid; i < 4 * TP; i += blockDim.x) rs[i * RP + C] = 1.f;  // the bias row of r

    auto build_table = [&](int t, int slot) {
        if (tid < TP) {
            const int qc = t * TP + tid;
            int pix = -1, flat = -1, flags = 0;
            int cst[4] = {-1, -1, -1, -1};
            if (qc < ncell) {
                const int ly = r0 + qc / w, lx = qc - (qc / w) * w;
                pix = (y0 + ly) * D.Wc + x0 + lx;
#pragma unroll
                for (int dd = 0; dd < 4; ++dd) {
                    cst[dd] = stash_pos(h, w, ly, lx, dd);
                    const bool lok = (dd & 1) ? lx < w - 1 : lx > 0;  // left predecessor (y, x - sx)
                    const bool uok = (dd & 2) ? ly < h - 1 : ly > 0;  // upper predecessor (y - sy, x)
                    flags |= (lok ? 1 : 0) << (2 * dd) | (uok ? 2 : 0) << (2 * dd);
                }
                const int qy = y0 + ly - ry0, qx = x0 + lx - rx0;
                if (qy < rh && qx < rw) flat = (int)(D.flat_off[e] + qy * rw + qx);
            }
            tpix[slot * TP + tid] = pix;
            tflat[slot * TP + tid] = flat;
            tflag[slot * TP + tid] = flags;
#pragma unroll
            for (int dd = 0; dd < 4; ++dd) tcst[(slot * 4 + dd) * TP + tid] = cst[dd];
        }
    };

    // this wave's direction: its h plane and its gate gradients, each one 32-bit range
    const __amdgpu_buffer_rsrc_t rH = rsrc(hdirs + d * plane, plane * 4);
    const __amdgpu_buffer_rsrc_t rA4 = rsrc(dA + (int64_t)d * D.T * 4 * H, (int64_t)D.T * 16 * H);
    const __amdgpu_buffer_rsrc_t rA1 = rsrc(dA + z1_offset(D.T, H) + (int64_t)d * D.T * H, (int64_t)D.T * 4 * H);
    const __amdgpu_buffer_rsrc_t rX = rsrc(xc, (int64_t)D.Hc * D.Wc * C * XB);

    // staged values of one tile for this thread's direction
    HV vh[S::NHL];
    f32x4 vd4[S::ND4];
    HV vd1[S::ND1];
    float vx[S::NXL];
    auto issue_loads = [&](int slot) {
        const int* pix = tpix + slot * TP;
        const int* flg = tflag + slot * TP;
        const int* cst = tcst + (slot * 4 + d) * TP;
#pragma unroll
        for (int i = 0; i < S::NHL; ++i) {
            const int idx = td + i * NTH;  // (cell, part, vector) of [TP][2][H / VH]
            int off = kOOBw;
            if (idx < TP * 2 * H / VH) {
                const int c = idx / (2 * H / VH), rem = idx - c * (2 * H / VH);
                const int up = rem / (H / VH), kv = rem - up * (H / VH);
                const int p = pix[c], fl = flg[c] >> (2 * d);
                const int src = up ? ((fl & 2) ? p + ((d & 2) ? D.Wc : -D.Wc) : -1)
                                   : ((fl & 1) ? p + ((d & 1) ? 1 : -1) : -1);
                if (p >= 0 && src >= 0) off = (src * H + kv * VH) * 4;
            }
            vh[i] = vload<VH>(rH, off);
        }
#pragma unroll
        for (int i = 0; i < S::ND4; ++i) {
            const int idx = td + i * NTH;  // (cell, unit)
            int off = kOOBw;
            if (idx < TP * H) {
                const int c = idx / H, k = idx - c * H;
                if (cst[c] >= 0) off = ((cell0 + cst[c]) * H + k) * 16;
            }
            vd4[i] = vload<4>(rA4, off);
        }
#pragma unroll
        for (int i = 0; i < S::ND1; ++i) {
            const int idx = td + i * NTH;  // (cell, vector of units)
            int off = kOOBw;
            if (idx < TP * H / VH) {
                const int c = idx / (H / VH), kv = idx - c * (H / VH);
                if (cst[c] >= 0) off = ((cell0 + cst[c]) * H + kv * VH) * 4;
            }
            vd1[i] = vload<VH>(rA1, off);
        }
#pragma unroll
        for (int i = 0; i < S::NXL; ++i) {
            const int idx = td + i * NTH;  // (cell, channel)
            int off = kOOBw;
            if (idx < TP * C) {
                const int c = idx / C, k = idx - c * C;
                if (pix[c] >= 0) off = (pix[c] * C + k) * XB;
            }
            if constexpr (BF16) vx[i] = __uint_as_float((uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rX, off, 0, 0) << 16);
            else vx[i] = bld(rX, off);
        }
    };
    auto write_lds = [&]() {
        float* rsd = rs + d * TP * RP;
        float* dad = das + d * TP * DS;
#pragma unroll
        for (int i = 0; i < S::NHL; ++i) {
            const int idx = td + i * NTH;
            if (idx < TP * 2 * H / VH) {
                const int c = idx / (2 * H / VH), rem = idx - c * (2 * H / VH);
                const int up = rem / (H / VH), kv = rem - up * (H / VH);
#pragma unroll
                for (int j = 0; j < VH; ++j) rsd[c * RP + C + 1 + up * H + kv * VH + j] = vget<VH>(vh[i], j);
            }
        }
#pragma unroll
        for (int i = 0; i < S::ND4; ++i) {
            const int idx = td + i * NTH;
            if (idx < TP * H) {
                const int c = idx / H, k = idx - c * H;
#pragma unroll
                for (int g = 0; g < 4; ++g) dad[c * DS + 4 * k + g] = vd4[i][g];
            }
        }
#pragma unroll
        for (int i = 0; i < S::ND1; ++i) {
            const int idx = td + i * NTH;
            if (idx < TP * H / VH) {
                const int c = idx / (H / VH), kv = idx - c * (H / VH);
#pragma unroll
                for (int j = 0; j < VH; ++j) dad[c * DS + 4 * H + kv * VH + j] = vget<VH>(vd1[i], j);
            }
        }
#pragma unroll
        for (int i = 0; i < S::NXL; ++i) {
            const int idx = td + i * NTH;
            if (idx < TP * C) {
                const int c = idx / C, k = idx - c * C;
                rsd[c * RP + k] = vx[i];
            }
        }
    };

    // B fragments of the r^T da product: LDS offset of gate-unit column n = 16 (nt0 + j) + i16 within a da row
    int bo[NTW];
#pragma unroll
    for (int j = 0; j < NTW; ++j) {
        const int n = 16 * (nt0 + j) + i16;
        const int g = n / H, k = n - g * H;
        bo[j] = (nt0 + j < NT && n < G) ? (g < 4 ? 4 * k + g : 4 * H + k) : G;  // column G of a row is zero
    }
    // dx: B = Wx[d]^T, rows n = 4 ks + q, column c = i16; kept in registers when one wave serves the
    // direction, read from the (cached) weights otherwise
    constexpr bool BREG = WPD == 1;
    float bwx[BREG ? KX : 1];
    auto wx_b = [&](int ks) {
        const int n = 4 * ks + q;
        return (i16 < C && n < G) ? Wx[((int64_t)d * C + i16) * G + n] : 0.f;
    };
    if constexpr (BREG) {
#pragma unroll
        for (int ks = 0; ks < KX; ++ks) bwx[ks] = wx_b(ks);
    }

    f32x4 acc[MT][NTW];
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int j = 0; j < NTW; ++j) acc[m][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    build_table(0, 0);
    __syncthreads();
    issue_loads(0);
    for (int t = 0; t < ntiles; ++t) {
        const int slot = t % 3;
        write_lds();
        if (t + 1 < ntiles) build_table(t + 1, (t + 1) % 3);
        __syncthreads();
        if (t + 1 < ntiles) issue_loads((t + 1) % 3);
        const float* rsd = rs + d * TP * RP;
        const float* dad = das + d * TP * DS;
#pragma unroll
        for (int ks = 0; ks < TP / 4; ++ks) {
            const int c = 4 * ks + q;
            float af[MT], bf[NTW];
#pragma unroll
            for (int m = 0; m < MT; ++m) af[m] = rsd[c * RP + 16 * m + i16];
#pragma unroll
            for (int j = 0; j < NTW; ++j) bf[j] = dad[c * DS + bo[j]];
#pragma unroll
            for (int m = 0; m < MT; ++m)
#pragma unroll
                for (int j = 0; j < NTW; ++j)
                    if (nt0 + j < NT) acc[m][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(af[m], bf[j], acc[m][j], 0, 0, 0);
        }
        // dx of this direction for the tile's cells: 16-cell M tiles shared out over the direction's waves
        for (int m2 = sub; m2 < TP / 16; m2 += WPD) {
            const float* arow = dad + (16 * m2 + i16) * DS;
            f32x4 dacc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KX; ++ks) {
                const int n = 4 * ks + q;
                const int g = n / H, k = n - g * H;
                const float av = n < G ? arow[g < 4 ? 4 * k + g : 4 * H + k] : 0.f;
                dacc = __builtin_amdgcn_mfma_f32_16x16x4f32(av, BREG ? bwx[BREG ? ks : 0] : wx_b(ks), dacc, 0, 0, 0);
            }
#pragma unroll
            for (int r = 0; r < 4; ++r)
                if (i16 < C) dxs[(d * TP + 16 * m2 + 4 * q + r) * C + i16] = dacc[r];
        }
        __syncthreads();
        {
            const int* pix = tpix + slot * TP;
            const int* flat = tflat + slot * TP;
            for (int o = tid; o < TP * C; o += blockDim.x) {
                const int c = o / C, chn = o - c * C;
                if (pix[c] < 0) continue;
                const float v = ((dxs[(0 * TP + c) * C + chn] + dxs[(1 * TP + c) * C + chn]) +
                                 dxs[(2 * TP + c) * C + chn]) + dxs[(3 * TP + c) * C + chn];
                if (dx_flat && flat[c] >= 0) dx_flat[(int64_t)flat[c] * C + chn] = v;
                if (dx_canvas) dx_canvas[(int64_t)pix[c] * C + chn] = flat[c] >= 0 ? v : 0.f;
            }
        }
    }
    // partial sums of this chunk: part[chunk][d][R][G]
    float* out = part + ((int64_t)ch * 4 + d) * R * G;
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

template <bool BF16, int C, int H>
size_t wg2_lds() {
    using S = WgShape<C, H>;
    return 4 * ((size_t)4 * TP * S::RP + (size_t)4 * TP * S::DS + (size_t)4 * TP * C + (size_t)3 * TP * 7);
}

typedef void (*Wg2Kernel)(Dev, const void*, const float*, const float*, const float*, float*, float*, float*);

struct Wg2Entry {
    bool bf16;
    int C, H, threads;
    size_t lds;
    Wg2Kernel k;
};
#define MDL_WG2(bf, c, h) {bf, c, h, 256 * WgShape<c, h>::WPD, wg2_lds<bf, c, h>(), k_wgrad2<bf, c, h>}
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
                         hipStream_t st) {
    const Wg2Entry* m = wg2_entry(C, H, dtype != 0);
    if (!m) return hipErrorInvalidValue;
    hipLaunchKernelGGL(m->k, dim3((unsigned)D.nchunks), dim3(m->threads), m->lds, st, D, x_canvas, h_dirs, dA, Wx,
                       part, dx_flat, dx_canvas);
    return hipGetLastError();
}

}  // namespace mdl
