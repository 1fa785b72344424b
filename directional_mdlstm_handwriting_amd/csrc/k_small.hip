// k_small.hip — wavefront kernels for small hidden sizes (H <= 10): the recurrence on the vector ALUs.
//
// Same schedule as the other wavefront kernels ("No Padding Please" §IV-A and RETURNN §4.2: all cells of a
// local anti-diagonal are independent; one workgroup per (example, direction) unit walks its diagonals,
// the backward in reverse order as "Single Stream Parallelization of Generalized LSTM-Like RNNs on a GPU"
// prescribes). With a few hidden units a 16-column matrix tile would be mostly padding, so here one thread
// owns one (diagonal position j, hidden unit k) element and computes its five gates from its own copy of
// unit k's weights (input projection x.Wx + b fused, recurrent product h_left.Ul + h_up.Uu), in fp32.
//
// Step structure shared with the matrix-core kernels: the loop is unrolled by four so every step is
// straight code; the step's global inputs (canvas pixels forward; the forward's factors and the upstream
// gradient backward) are prefetched three diagonals ahead into four register sets; loads and stores use
// raw buffer instructions with an out-of-range offset for a masked lane; a zero row in LDS stands in for
// a missing neighbour. One barrier per step: the forward double-buffers (h, c) of the diagonals, the
// backward double-buffers the gate gradients and the dc * f terms.
#include "kernels.h"
#include "devmath.h"

#include <type_traits>

namespace mdl {

namespace {

constexpr int kOOBs = 0x40000000;  // byte offset past every per-unit range used here (1 GiB)
constexpr int kPFs = 3;            // diagonals of prefetch ahead
constexpr int kSmallThreads = 1024;  // workgroup size bound of the H = 2 instances; H = 4 and 10 take 512

template <int N>
using ICs = std::integral_constant<int, N>;

// Diagonal s of an h x w unit: its length (0 outside [0, h + w - 1)) and its first row.
__device__ inline int sd_len(int h, int w, int s) {
    if (s < 0 || s >= h + w - 1) return 0;
    const int lo = s > w - 1 ? s - (w - 1) : 0;
    const int hi = s < h - 1 ? s : h - 1;
    return hi - lo + 1;
}
__device__ inline int sd_lo(int w, int s) { return s > w - 1 ? s - (w - 1) : 0; }

// Forward. Thread t owns element (j = t / H, k = t % H) of every diagonal; NP = blockDim / H positions.
// MAXT bounds the workgroup size (and so sets the register budget of unit k's weights).
template <int H, int C, bool BF16, int MAXT>
__global__ __launch_bounds__(MAXT) void k_fwd_small(Dev D, const void* __restrict__ xc,
                                                             const float* __restrict__ Wx,
                                                             const float* __restrict__ bias,
                                                             const float* __restrict__ Ul,
                                                             const float* __restrict__ Uu,
                                                             float* __restrict__ stash, float* __restrict__ hdirs) {
    constexpr int G = 5 * H;
    constexpr int XB = BF16 ? 2 : 4;
    const int u = D.units[blockIdx.x];
    const int e = u >> 2, d = u & 3;
    const int y0 = D.rect[4 * e], x0 = D.rect[4 * e + 1], h = D.rect[4 * e + 2], w = D.rect[4 * e + 3];
    const int tid = threadIdx.x;
    const int j = tid / H, k = tid - (tid / H) * H;
    const int NP = blockDim.x / H, ZR = NP;  // rows 0 .. NP-1: positions; ZR: zeros

    // unit k's weights, the gate order (i, f_l, f_u, o, g) along G
    float bz[5], wx[5][C], ul[5][H], uu[5][H];
#pragma unroll
    for (int g = 0; g < 5; ++g) {
        bz[g] = bias[(int64_t)d * G + g * H + k];
#pragma unroll
        for (int c = 0; c < C; ++c) wx[g][c] = Wx[((int64_t)d * C + c) * G + g * H + k];
#pragma unroll
        for (int q = 0; q < H; ++q) {
            ul[g][q] = Ul[((int64_t)d * H + q) * G + g * H + k];
            uu[g][q] = Uu[((int64_t)d * H + q) * G + g * H + k];
        }
    }
    // LDS: h and c of two diagonals, [2][NP + 1][HP] each (rows padded to whole 16-byte vectors, the
    // padding zero)
    constexpr int HP = (H + 3) / 4 * 4;
    extern __shared__ __align__(16) float sm[];
    const int RB = (NP + 1) * HP;  // floats of one buffer
    float* hb = sm;
    float* cb = sm + 2 * RB;
    for (int i = tid; i < 4 * RB; i += blockDim.x) sm[i] = 0.f;

    const int64_t base = (int64_t)d * D.T + D.cell_off[e];
    const int64_t cells = (int64_t)h * w;
    const __amdgpu_buffer_rsrc_t rX = rsrc(xc, (int64_t)D.Hc * D.Wc * C * XB);
    const __amdgpu_buffer_rsrc_t rS4 = rsrc(stash + base * 4 * H, cells * 16 * H);
    const __amdgpu_buffer_rsrc_t rS2 = rsrc(stash + z1_offset(D.T, H) + base * 4 * H, cells * 16 * H);
    const __amdgpu_buffer_rsrc_t rH = rsrc(hdirs + (int64_t)d * D.Hc * D.Wc * H, (int64_t)D.Hc * D.Wc * H * 4);
    const int S = h + w - 1;
    // cell (a, b) of the unit (b = s - a on diagonal s) sits at canvas (Y0 + SY a, X0 + SX b): its pixel is
    // PB + a PA + s PS
    const int SY = (d & 2) ? -1 : 1, SX = (d & 1) ? -1 : 1;
    const int Y0 = (d & 2) ? y0 + h - 1 : y0, X0 = (d & 1) ? x0 + w - 1 : x0;
    const int PB = Y0 * D.Wc + X0, PA = SY * D.Wc - SX, PS = SX;

    // input pixel of this thread's cell on diagonal s1 (zeros where absent)
    auto load_x = [&](int s1, float (&xv)[C]) {
        const int L1 = sd_len(h, w, s1);
        const int pix = PB + (sd_lo(w, s1 < 0 ? 0 : s1) + j) * PA + s1 * PS;
        const bool va = j < L1;
#pragma unroll
        for (int c = 0; c < C; ++c) {
            const int off = va ? (pix * C + c) * XB : kOOBs;
            if constexpr (BF16)
                xv[c] = __uint_as_float((uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rX, off, 0, 0) << 16);
            else
                xv[c] = bld(rX, off);
        }
    };
    float xs[4][C];
#pragma unroll
    for (int i = 0; i < kPFs; ++i) load_x(i, xs[i]);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the loop starts with nothing in flight
    __syncthreads();

    int st = 0;  // stash index of the first cell of diagonal s
    auto step = [&](int s, auto POSc) {
        constexpr int POS = decltype(POSc)::value;
        const int L = sd_len(h, w, s);
        load_x(s + kPFs, xs[(POS + kPFs) & 3]);
        __builtin_amdgcn_sched_barrier(0);  // keep the prefetch at the top of the step
        const int lo = sd_lo(w, s);
        const int dl = s >= w ? 1 : 0;
        const int Ml = L < s - lo ? L : s - lo;  // position j has a left predecessor iff j < Ml
        const int Tu = 1 - dl;                   // ... and an upper one iff Tu <= j < L
        const int rl = j < Ml ? j + dl : ZR;
        const int ru = (j >= Tu && j < L) ? j + dl - 1 : ZR;
        const float* hp = hb + ((s + 1) & 1) * RB;
        const float* cp = cb + ((s + 1) & 1) * RB;
        float hl[HP], hu[HP];
#pragma unroll
        for (int q4 = 0; q4 < HP / 4; ++q4) {
            const f32x4 vl = *reinterpret_cast<const f32x4*>(hp + rl * HP + 4 * q4);
            const f32x4 vu = *reinterpret_cast<const f32x4*>(hp + ru * HP + 4 * q4);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                hl[4 * q4 + i] = vl[i];
                hu[4 * q4 + i] = vu[i];
            }
        }
        const float cl = cp[rl * HP + k], cu = cp[ru * HP + k];
        // each gate as one chain of fused multiply-adds, or for larger H two (input and left predecessor;
        // upper predecessor) added at the end, halving the dependent chain
        float z[5];
#pragma unroll
        for (int g = 0; g < 5; ++g) {
            float a = bz[g], a2 = 0.f;
#pragma unroll
            for (int c = 0; c < C; ++c) a = __builtin_fmaf(xs[POS][c], wx[g][c], a);
#pragma unroll
            for (int q = 0; q < H; ++q) a = __builtin_fmaf(hl[q], ul[g][q], a);
            if constexpr (H >= 8) {
#pragma unroll
                for (int q = 0; q < H; ++q) a2 = __builtin_fmaf(hu[q], uu[g][q], a2);
                z[g] = a + a2;
            } else {
#pragma unroll
                for (int q = 0; q < H; ++q) a = __builtin_fmaf(hu[q], uu[g][q], a);
                z[g] = a;
            }
        }
        const float ig = sigm(z[0]), fl = sigm(z[1]), fu = sigm(z[2]), og = sigm(z[3]);
        const float gg = ftanh(z[4]);
        const float c = __builtin_fmaf(fl, cl, __builtin_fmaf(fu, cu, ig * gg));
        const float tc = ftanh(c);
        const float hv = og * tc;
        // positions past the diagonal write their own rows too: no later step reads them
        hb[(s & 1) * RB + j * HP + k] = hv;
        cb[(s & 1) * RB + j * HP + k] = c;
        const bool ok = j < L;
        const int el = (st + j) * H + k;
        bst(hv, rH, ok ? ((PB + (lo + j) * PA + s * PS) * H + k) * 4 : kOOBs);
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, f32x4{ig, fl, fu, og}), rS4,
                                               ok ? el * 16 : kOOBs, 0, 0);
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, f32x4{gg, tc, cl, cu}), rS2,
                                               ok ? el * 16 : kOOBs, 0, 0);
        st += L;
        __syncthreads();
    };
    int s = 0;
    for (; s + 4 <= S; s += 4) {
        step(s, ICs<0>{});
        step(s + 1, ICs<1>{});
        step(s + 2, ICs<2>{});
        step(s + 3, ICs<3>{});
    }
    if (s < S) step(s, ICs<0>{});
    if (s + 1 < S) step(s + 1, ICs<1>{});
    if (s + 2 < S) step(s + 2, ICs<2>{});
}

// Backward over the diagonals in reverse. For cell (a, b) on diagonal s, with successors R = (a, b+1) and
// D = (a+1, b) on s+1 (gate gradients da, terms dc f_l of R and dc f_u of D):
//     dh = dy + da(R) . Ul[k][:] + da(D) . Uu[k][:],  dc_in = (dc f_l)(R) + (dc f_u)(D)
//     tc = tanh c,  dc = dc_in + dh o (1 - tc^2)
//     da = [dc g i(1-i), dc c_l f_l(1-f_l), dc c_u f_u(1-f_u), dh tc o(1-o), dc i (1-g^2)]
// with c_l, c_u and tc = tanh c read from the forward's stash (SA, SB) with the gates.
template <int H, int MAXT>
__global__ __launch_bounds__(MAXT) void k_bwd_small(Dev D, const float* __restrict__ Ul,
                                                             const float* __restrict__ Uu,
                                                             const float* __restrict__ stash,
                                                             const float* __restrict__ dy_flat,
                                                             const float* __restrict__ dh_dirs,
                                                             float* __restrict__ dA) {
    constexpr int G = 5 * H;
    const int u = D.units[blockIdx.x];
    const int e = u >> 2, d = u & 3;
    const int y0 = D.rect[4 * e], x0 = D.rect[4 * e + 1], h = D.rect[4 * e + 2], w = D.rect[4 * e + 3];
    const int ry0 = D.real[4 * e], rx0 = D.real[4 * e + 1], rh = D.real[4 * e + 2], rw = D.real[4 * e + 3];
    const int tid = threadIdx.x;
    const int j = tid / H, k = tid - (tid / H) * H;
    const int NP = blockDim.x / H, ZR = NP;

    // unit k's rows of Ul[d] and Uu[d]: the weights from h_k of this cell to each gate column of the cell
    // that has it as left / upper predecessor
    constexpr int GP = (G + 3) / 4 * 4;  // gate-gradient row stride: whole 16-byte vectors, the padding zero
    float wl[GP], wu[GP];
#pragma unroll
    for (int n = 0; n < GP; ++n) {
        wl[n] = n < G ? Ul[((int64_t)d * H + k) * G + n] : 0.f;
        wu[n] = n < G ? Uu[((int64_t)d * H + k) * G + n] : 0.f;
    }
    // LDS, each [2][NP + 1][.]: gate gradients (GP per row), dc f_l and dc f_u (H per row)
    extern __shared__ __align__(16) float sm[];
    const int RG = (NP + 1) * GP, RH = (NP + 1) * H;
    float* dab = sm;
    float* dcl = dab + 2 * RG;
    float* dcu = dcl + 2 * RH;
    for (int i = tid; i < 2 * RG + 4 * RH; i += blockDim.x) sm[i] = 0.f;

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
    const int S = h + w - 1;
    // Cell (a, b) sits at canvas (Y0 + SY a, X0 + SX b). Its upstream gradient's byte offset is
    // UB + a UA + s US + 4 k: on the canvas plane for a per-direction gradient, else in the example's flat
    // real-pixel block, where the cell must also lie in the real region.
    const int SY = (d & 2) ? -1 : 1, SX = (d & 1) ? -1 : 1;
    const int Y0 = (d & 2) ? y0 + h - 1 : y0, X0 = (d & 1) ? x0 + w - 1 : x0;
    const int H4 = 4 * H;
    const int rowlen = per_dir ? D.Wc : rw;
    const int UY = per_dir ? Y0 : Y0 - ry0, UX = per_dir ? X0 : X0 - rx0;
    const int UA = SY * rowlen * H4 - SX * H4, US = SX * H4;
    const int UB = (UY * rowlen + UX) * H4 + 4 * k;
    // real region in unit coordinates: a in [ar0, ar1), b in [br0, br1)
    const int ar0 = (d & 2) ? h - (ry0 - y0) - rh : ry0 - y0, ar1 = ar0 + rh;
    const int br0 = (d & 1) ? w - (rx0 - x0) - rw : rx0 - x0, br1 = br0 + rw;

    struct Fw {
        f32x4 fa, fb;  // the forward's values (SA, SB)
        float dy;
    };
    // forward values of this thread's element on diagonal s1 (stash index st1 of its first cell)
    auto load_f = [&](int s1, int st1, Fw& f) {
        const int L1 = sd_len(h, w, s1);
        const int lo1 = sd_lo(w, s1 < 0 ? 0 : s1);
        const bool ok = j < L1;
        const int el = st1 * H + j * H + k;
        f.fa = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rS4, ok ? el * 16 : kOOBs, 0, 0));
        f.fb = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rS2, ok ? el * 16 : kOOBs, 0, 0));
        const int a = lo1 + j, b = s1 - a;
        const bool vy = ok & (per_dir | ((a >= ar0) & (a < ar1) & (b >= br0) & (b < br1)));
        f.dy = bld(rU, vy ? UB + a * UA + s1 * US : kOOBs);
    };

    Fw fs[4];
    int st = (int)cells - 1;  // stash index of the first cell of diagonal s (diagonal S - 1 is the last cell)
    int stz = st;             // ... of the prefetch diagonal
#pragma unroll
    for (int i = 0; i < kPFs; ++i) {
        load_f(S - 1 - i, stz, fs[i]);
        stz -= sd_len(h, w, S - 2 - i);
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    __syncthreads();

    // diagonal s at position POS = (S - 1 - s) mod 4: prefetch set POS holds diagonal s and (POS + kPFs) & 3
    // is refilled for diagonal s - kPFs
    auto step = [&](int s, auto POSc) {
        constexpr int POS = decltype(POSc)::value;
        const int L = sd_len(h, w, s), L1 = sd_len(h, w, s + 1);
        load_f(s - kPFs, stz, fs[(POS + kPFs) & 3]);
        stz -= sd_len(h, w, s - kPFs - 1);
        __builtin_amdgcn_sched_barrier(0);
        __syncthreads();
        const Fw& f = fs[POS];
        const int dn = s >= w - 1 ? 1 : 0;  // successors of position j: right j - dn, down j + 1 - dn
        const int rr = j >= dn ? j - dn : ZR;
        const int rd = j + 1 - dn < L1 ? j + 1 - dn : ZR;
        const float* dar = dab + ((s + 1) & 1) * RG;
        // dh as four partial sums over the two successors' gate gradients
        float p0 = f.dy, p1 = 0.f, p2 = 0.f, p3 = 0.f;
#pragma unroll
        for (int n4 = 0; n4 < GP / 4; ++n4) {
            const f32x4 vr = *reinterpret_cast<const f32x4*>(dar + rr * GP + 4 * n4);
            const f32x4 vd = *reinterpret_cast<const f32x4*>(dar + rd * GP + 4 * n4);
            p0 = __builtin_fmaf(vr[0], wl[4 * n4], p0);
            p1 = __builtin_fmaf(vr[1], wl[4 * n4 + 1], p1);
            p0 = __builtin_fmaf(vr[2], wl[4 * n4 + 2], p0);
            p1 = __builtin_fmaf(vr[3], wl[4 * n4 + 3], p1);
            p2 = __builtin_fmaf(vd[0], wu[4 * n4], p2);
            p3 = __builtin_fmaf(vd[1], wu[4 * n4 + 1], p3);
            p2 = __builtin_fmaf(vd[2], wu[4 * n4 + 2], p2);
            p3 = __builtin_fmaf(vd[3], wu[4 * n4 + 3], p3);
        }
        const float dh = (p0 + p1) + (p2 + p3);
        const float dcin = dcl[((s + 1) & 1) * RH + rr * H + k] + dcu[((s + 1) & 1) * RH + rd * H + k];
        f32x4 ka, kb;
        bwd_factors(f.fa, f.fb, ka, kb);
        const float dc = __builtin_fmaf(dh, kb[1], dcin);
        const float d0 = dc * ka[0], d1 = dc * ka[1], d2 = dc * ka[2], d3 = dh * ka[3], d4 = dc * kb[0];
        // positions past the diagonal write their own rows: no step reads them as successors
        float* daw = dab + (s & 1) * RG + j * GP + k;
        daw[0] = d0;
        daw[H] = d1;
        daw[2 * H] = d2;
        daw[3 * H] = d3;
        daw[4 * H] = d4;
        dcl[(s & 1) * RH + j * H + k] = dc * kb[2];
        dcu[(s & 1) * RH + j * H + k] = dc * kb[3];
        const bool ok = j < L;
        const int el = st * H + j * H + k;
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, f32x4{d0, d1, d2, d3}), rA4,
                                               ok ? el * 16 : kOOBs, 0, 0);
        bst(d4, rA1, ok ? el * 4 : kOOBs);
        st -= sd_len(h, w, s - 1);
    };
    int s = S - 1;
    for (; s - 3 >= 0; s -= 4) {
        step(s, ICs<0>{});
        step(s - 1, ICs<1>{});
        step(s - 2, ICs<2>{});
        step(s - 3, ICs<3>{});
    }
    if (s >= 0) step(s, ICs<0>{});
    if (s - 1 >= 0) step(s - 1, ICs<1>{});
    if (s - 2 >= 0) step(s - 2, ICs<2>{});
}

typedef void (*FwdSmallKernel)(Dev, const void*, const float*, const float*, const float*, const float*, float*,
                               float*);
typedef void (*BwdSmallKernel)(Dev, const float*, const float*, const float*, const float*, const float*, float*);

struct SmallFwd {
    int H, C;
    bool bf16;
    int maxt;
    FwdSmallKernel k;
};
#define MDL_SF(h, c, bf, t) {h, c, bf, t, k_fwd_small<h, c, bf, t>}
const SmallFwd kSmallFwd[] = {MDL_SF(2, 4, false, kSmallThreads), MDL_SF(4, 1, false, 512),
                              MDL_SF(2, 1, false, kSmallThreads), MDL_SF(4, 4, false, 512),
                              MDL_SF(10, 6, false, 512)};
#undef MDL_SF
struct SmallBwd {
    int H, maxt;
    BwdSmallKernel k;
};
const SmallBwd kSmallBwd[] = {{2, kSmallThreads, k_bwd_small<2, kSmallThreads>},
                              {4, 512, k_bwd_small<4, 512>},
                              {10, 512, k_bwd_small<10, 512>}};

// threads: one per (position, unit) of the widest diagonal (the last wave may be partial)
int small_threads(int H, int Lmax) { return (Lmax < 1 ? 1 : Lmax) * H; }
int small_positions(int H, int Lmax) { return small_threads(H, Lmax) / H; }

const SmallFwd* small_fwd_entry(int H, int C, int dtype, int Lmax) {
    const int t = small_threads(H, Lmax);
    for (const auto& m : kSmallFwd)
        if (m.H == H && m.C == C && m.bf16 == (dtype != 0)) return t <= m.maxt ? &m : nullptr;
    return nullptr;
}
const SmallBwd* small_bwd_entry(int H, int Lmax) {
    const int t = small_threads(H, Lmax);
    for (const auto& m : kSmallBwd)
        if (m.H == H) return t <= m.maxt ? &m : nullptr;
    return nullptr;
}

}  // namespace

bool small_fwd_supported(int H, int C, int dtype, int Lmax) { return small_fwd_entry(H, C, dtype, Lmax) != nullptr; }

bool small_bwd_supported(int H, int Lmax) { return small_bwd_entry(H, Lmax) != nullptr; }

size_t small_fwd_lds(int H, int Lmax) {
    return sizeof(float) * 4 * (size_t)(small_positions(H, Lmax) + 1) * ((H + 3) / 4 * 4);
}

size_t small_bwd_lds(int H, int Lmax) {
    const size_t rows = small_positions(H, Lmax) + 1;
    return sizeof(float) * (2 * rows * ((5 * H + 3) / 4 * 4) + 4 * rows * H);
}

hipError_t launch_fwd_small(const Dev& D, const void* x_canvas, int dtype, int C, int H, const float* Wx,
                            const float* b, const float* Ul, const float* Uu, float* stash, float* h_dirs,
                            hipStream_t st) {
    const SmallFwd* m = small_fwd_entry(H, C, dtype, D.max_diag);
    if (!m) return hipErrorInvalidValue;
    launch(m->k, dim3(4 * D.n), dim3(small_threads(H, D.max_diag)), small_fwd_lds(H, D.max_diag), st, D, x_canvas,
           Wx, b, Ul, Uu, stash, h_dirs);
    return hipGetLastError();
}

hipError_t launch_bwd_small(const Dev& D, int H, const float* Ul, const float* Uu, const float* stash,
                            const float* dy_flat, const float* dh_dirs, float* dA, hipStream_t st) {
    const SmallBwd* m = small_bwd_entry(H, D.max_diag);
    if (!m) return hipErrorInvalidValue;
    launch(m->k, dim3(4 * D.n), dim3(small_threads(H, D.max_diag)), small_bwd_lds(H, D.max_diag), st, D, Ul, Uu,
           stash, dy_flat, dh_dirs, dA);
    return hipGetLastError();
}

}  // namespace mdl
