// k_skew.hip — the pages' own schedule of the recurrence: column steps over the input-skewed canvas.
//
// "No Padding Please" §IV-A (Figure 3) skews the whole packed canvas, row i shifted right by i, so that in
// each direction the cells a step can compute together are one column of the skewed grid: the canvas cells
// with y' + x' = k (y', x' counted along the direction's scan). A pass then takes Hc + Wc - 1 dependent
// column steps over the whole canvas, and every cell of the skewed grid is computed, padding and separators
// included, the mask (§V) zeroing what does not belong to an example. RETURNN §4.2 runs such a diagonal
// recurrence as one kernel launch per diagonal. These kernels do the same: one launch per skewed column,
// all four directions in one grid, every column cell computed (gate arithmetic on zero inputs where the
// column cell is padding) and only the example cells stored. Results are the same cell values as the local
// schedule's; the stash, the projection and the gate gradients keep that schedule's per-example
// diagonal-major layout, so the weight gradients are computed by the same kernels afterwards.
//
// One thread per (column cell, hidden unit): it reads its predecessors' h from the canvas planes and their
// memory states from the stash, and the block's direction weights from LDS; fp32 throughout.
#include "kernels.h"
#include "devmath.h"
#include "layout.h"

namespace mdl {

namespace {

constexpr int SK_THREADS = 256;

struct SkewCell {
    bool real;
    int y, x, e, a, b;
};

// the column cell of row y on skewed column k, direction d
__device__ inline SkewCell skew_cell(const Dev& D, int d, int k, int y) {
    SkewCell c{false, y, 0, -1, 0, 0};
    const int yy = (d & 2) ? D.Hc - 1 - y : y;  // row counted along the scan
    const int xx = k - yy;
    if (y >= D.Hc || xx < 0 || xx >= D.Wc) return c;  // skew padding
    c.x = (d & 1) ? D.Wc - 1 - xx : xx;
    const int e = D.eid[(int64_t)y * D.Wc + c.x];
    if (e < 0) return c;  // separator or unused canvas
    const int y0 = D.rect[4 * e], x0 = D.rect[4 * e + 1], h = D.rect[4 * e + 2], w = D.rect[4 * e + 3];
    c.e = e;
    c.a = (d & 2) ? y0 + h - 1 - y : y - y0;
    c.b = (d & 1) ? x0 + w - 1 - c.x : c.x - x0;
    c.real = true;
    return c;
}

// diagonal-major position of direction-local cell (a, b) of example e, within direction d's stash
__device__ inline int64_t skew_index(const Dev& D, int d, int e, int a, int b) {
    const int h = D.rect[4 * e + 2], w = D.rect[4 * e + 3];
    const int s = a + b;
    return (int64_t)d * D.T + D.cell_off[e] + dg_start(h, w, s) + a - dg_lo(h, w, s);
}

// Forward column step k. Z: the projection x.Wx + b (Z4 | Z1 layout); stash and h_dirs out.
template <int H>
__global__ __launch_bounds__(SK_THREADS) void k_skew_fwd(Dev D, int k, const float* __restrict__ Ul,
                                                         const float* __restrict__ Uu, const float* __restrict__ Z,
                                                         float* __restrict__ stash, float* __restrict__ hdirs) {
    constexpr int G = 5 * H;
    const int d = blockIdx.y;
    __shared__ float U[2 * H * G];  // rows 0..H-1: Ul[d], rows H..2H-1: Uu[d]
    for (int i = threadIdx.x; i < H * G; i += blockDim.x) {
        U[i] = Ul[(int64_t)d * H * G + i];
        U[H * G + i] = Uu[(int64_t)d * H * G + i];
    }
    __syncthreads();
    const int item = blockIdx.x * blockDim.x + threadIdx.x;
    const int y = item / H, kk = item - y * H;
    const SkewCell c = skew_cell(D, d, k, y);
    const int sx = (d & 1) ? -1 : 1, sy = (d & 2) ? -1 : 1;
    const uint8_t bits = c.real ? D.border[(int64_t)y * D.Wc + c.x] : 0;
    const bool hasL = bits & (sx > 0 ? 1 : 2), hasU = bits & (sy > 0 ? 4 : 8);
    const float* Hd = hdirs + (int64_t)d * D.Hc * D.Wc * H;
    const float* hl = Hd + ((int64_t)y * D.Wc + c.x - sx) * H;
    const float* hu = Hd + ((int64_t)(y - sy) * D.Wc + c.x) * H;
    const float* S2 = stash + z1_offset(D.T, H);
    const int64_t ic = c.real ? skew_index(D, d, c.e, c.a, c.b) : 0;
    const float cl = hasL ? S2[(skew_index(D, d, c.e, c.a, c.b - 1) * H + kk) * 2 + 1] : 0.f;
    const float cu = hasU ? S2[(skew_index(D, d, c.e, c.a - 1, c.b) * H + kk) * 2 + 1] : 0.f;
    float acc[5];
#pragma unroll
    for (int g = 0; g < 4; ++g) acc[g] = c.real ? Z[(ic * H + kk) * 4 + g] : 0.f;
    acc[4] = c.real ? Z[z1_offset(D.T, H) + ic * H + kk] : 0.f;
    for (int q = 0; q < H; ++q) {
        const float vl = hasL ? hl[q] : 0.f, vu = hasU ? hu[q] : 0.f;
#pragma unroll
        for (int g = 0; g < 5; ++g) acc[g] += vl * U[q * G + g * H + kk] + vu * U[(H + q) * G + g * H + kk];
    }
    const float ig = sigm(acc[0]), fl = sigm(acc[1]), fu = sigm(acc[2]), og = sigm(acc[3]);
    const float gg = ftanh(acc[4]);
    const float cv = fl * cl + fu * cu + ig * gg;
    const float hv = og * ftanh(cv);
    if (c.real) {  // the mask: only example cells are kept
        hdirs[(int64_t)d * D.Hc * D.Wc * H + ((int64_t)y * D.Wc + c.x) * H + kk] = hv;
        *reinterpret_cast<f32x4*>(stash + (ic * H + kk) * 4) = f32x4{ig, fl, fu, og};
        *reinterpret_cast<f32x2*>(stash + z1_offset(D.T, H) + (ic * H + kk) * 2) = f32x2{gg, cv};
    }
}

// Backward column step k (columns in reverse). dcb [4][T][H][2]: (dc f_l, dc f_u) of every cell, what it sends
// to its left and upper predecessors; dA out in the local schedule's layout.
template <int H>
__global__ __launch_bounds__(SK_THREADS) void k_skew_bwd(Dev D, int k, const float* __restrict__ Ul,
                                                         const float* __restrict__ Uu, const float* __restrict__ stash,
                                                         const float* __restrict__ dy_flat,
                                                         const float* __restrict__ dh_dirs, float* __restrict__ dA,
                                                         float* __restrict__ dcb) {
    constexpr int G = 5 * H;
    const int d = blockIdx.y;
    __shared__ float UT[2 * H * G];  // UT[kk][n] = Ul[d][kk][n], then Uu[d]
    for (int i = threadIdx.x; i < H * G; i += blockDim.x) {
        UT[i] = Ul[(int64_t)d * H * G + i];
        UT[H * G + i] = Uu[(int64_t)d * H * G + i];
    }
    __syncthreads();
    const int item = blockIdx.x * blockDim.x + threadIdx.x;
    const int y = item / H, kk = item - y * H;
    const SkewCell c = skew_cell(D, d, k, y);
    const int sx = (d & 1) ? -1 : 1, sy = (d & 2) ? -1 : 1;
    const uint8_t bits = c.real ? D.border[(int64_t)y * D.Wc + c.x] : 0;
    const bool hasL = bits & (sx > 0 ? 1 : 2), hasU = bits & (sy > 0 ? 4 : 8);
    const bool hasR = bits & (sx > 0 ? 2 : 1), hasD = bits & (sy > 0 ? 8 : 4);  // successors
    const float* S2 = stash + z1_offset(D.T, H);
    const int64_t ic = c.real ? skew_index(D, d, c.e, c.a, c.b) : 0;
    const int64_t iR = hasR ? skew_index(D, d, c.e, c.a, c.b + 1) : 0;
    const int64_t iD = hasD ? skew_index(D, d, c.e, c.a + 1, c.b) : 0;
    float dh = 0.f;
    if (c.real) {
        if (dh_dirs) {
            dh = dh_dirs[(int64_t)d * D.Hc * D.Wc * H + ((int64_t)y * D.Wc + c.x) * H + kk];
        } else {
            const int ry0 = D.real[4 * c.e], rx0 = D.real[4 * c.e + 1], rh = D.real[4 * c.e + 2], rw = D.real[4 * c.e + 3];
            const int ly = y - ry0, lx = c.x - rx0;
            if (ly >= 0 && lx >= 0 && ly < rh && lx < rw) dh = dy_flat[(D.flat_off[c.e] + (int64_t)ly * rw + lx) * H + kk];
        }
    }
    const float* A1 = dA + z1_offset(D.T, H);
    for (int g = 0; g < 5; ++g)
        for (int j = 0; j < H; ++j) {
            const int n = g * H + j;
            const float vr = hasR ? (g < 4 ? dA[(iR * H + j) * 4 + g] : A1[iR * H + j]) : 0.f;
            const float vd = hasD ? (g < 4 ? dA[(iD * H + j) * 4 + g] : A1[iD * H + j]) : 0.f;
            dh += vr * UT[kk * G + n] + vd * UT[(H + kk) * G + n];
        }
    const float dcin = (hasR ? dcb[(iR * H + kk) * 2] : 0.f) + (hasD ? dcb[(iD * H + kk) * 2 + 1] : 0.f);
    const f32x4 g4 = c.real ? *reinterpret_cast<const f32x4*>(stash + (ic * H + kk) * 4) : f32x4{0.f, 0.f, 0.f, 0.f};
    const f32x2 g2 = c.real ? *reinterpret_cast<const f32x2*>(S2 + (ic * H + kk) * 2) : f32x2{0.f, 0.f};
    const float cl = hasL ? S2[(skew_index(D, d, c.e, c.a, c.b - 1) * H + kk) * 2 + 1] : 0.f;
    const float cu = hasU ? S2[(skew_index(D, d, c.e, c.a - 1, c.b) * H + kk) * 2 + 1] : 0.f;
    const float ig = g4[0], fl = g4[1], fu = g4[2], og = g4[3], gg = g2[0], cv = g2[1];
    const float tc = ftanh(cv);
    const float dov = dh * tc;
    const float dc = dcin + dh * og * (1.f - tc * tc);
    const float d0 = dc * gg * ig * (1.f - ig);
    const float d1 = dc * cl * fl * (1.f - fl);
    const float d2 = dc * cu * fu * (1.f - fu);
    const float d3 = dov * og * (1.f - og);
    const float d4 = dc * ig * (1.f - gg * gg);
    if (c.real) {
        *reinterpret_cast<f32x4*>(dA + (ic * H + kk) * 4) = f32x4{d0, d1, d2, d3};
        dA[z1_offset(D.T, H) + ic * H + kk] = d4;
        *reinterpret_cast<f32x2*>(dcb + (ic * H + kk) * 2) = f32x2{dc * fl, dc * fu};
    }
}

typedef void (*SkewFwdK)(Dev, int, const float*, const float*, const float*, float*, float*);
typedef void (*SkewBwdK)(Dev, int, const float*, const float*, const float*, const float*, const float*, float*,
                         float*);
struct SkewEntry {
    int H;
    SkewFwdK fwd;
    SkewBwdK bwd;
};
const SkewEntry kSkew[] = {{4, k_skew_fwd<4>, k_skew_bwd<4>}, {16, k_skew_fwd<16>, k_skew_bwd<16>}};

const SkewEntry* skew_entry(int H) {
    for (const auto& m : kSkew)
        if (m.H == H) return &m;
    return nullptr;
}

}  // namespace

bool skew_supported(int H) { return skew_entry(H) != nullptr; }

int skew_columns(const Dev& D) { return D.Hc + D.Wc - 1; }

hipError_t launch_skew_fwd(const Dev& D, int H, const float* Ul, const float* Uu, const float* Z, float* stash,
                           float* h_dirs, hipStream_t st) {
    const SkewEntry* m = skew_entry(H);
    if (!m) return hipErrorInvalidValue;
    const dim3 grid((unsigned)(((int64_t)D.Hc * H + SK_THREADS - 1) / SK_THREADS), 4);
    for (int k = 0; k < skew_columns(D); ++k) {
        launch(m->fwd, grid, dim3(SK_THREADS), 0, st, D, k, Ul, Uu, Z, stash, h_dirs);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

hipError_t launch_skew_bwd(const Dev& D, int H, const float* Ul, const float* Uu, const float* stash,
                           const float* dy_flat, const float* dh_dirs, float* dA, float* dcb, hipStream_t st) {
    const SkewEntry* m = skew_entry(H);
    if (!m) return hipErrorInvalidValue;
    const dim3 grid((unsigned)(((int64_t)D.Hc * H + SK_THREADS - 1) / SK_THREADS), 4);
    for (int k = skew_columns(D) - 1; k >= 0; --k) {
        launch(m->bwd, grid, dim3(SK_THREADS), 0, st, D, k, Ul, Uu, stash, dy_flat, dh_dirs, dA, dcb);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace mdl
