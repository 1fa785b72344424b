// k_proj.hip — input projection of every computed cell for all four directions.
//
// "No Padding Please", §IV-B: the five input matrices (input node, input gate,
// two forget gates, output gate) depend only on the input and are computed
// together, as one 1x1 convolution; RETURNN §4.2: the non-recurrent part of
// the LSTM is one matrix product for the whole mini-batch. Here it is one
// GEMM per 16-cell tile,
//     Z[d][cell][n] = sum_c x[cell][c] * Wx[d][c][n] + b[d][n],
// on the matrix cores (v_mfma_f32_16x16x4_f32: A 16 cells x 4 channels,
// B 4 channels x 16 gate columns, fp32 products and accumulation). The cell's
// pre-activations are written at its position in each direction's
// diagonal-major order (layouts Z4 / Z1), so the wavefront kernel reads each
// anti-diagonal contiguously.
// With C <= 20 input channels the kernel is bound by writing Z (5H floats per
// cell and direction), not by the matrix cores.
#include "kernels.h"

namespace mdl {

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

template <typename XT> __device__ inline float to_f32(XT v);
template <> __device__ inline float to_f32<float>(float v) { return v; }
template <> __device__ inline float to_f32<uint16_t>(uint16_t v) { return __uint_as_float(((uint32_t)v) << 16); }

// 256 threads = 4 waves; each wave owns 16 consecutive computed cells (cell
// order: example after example, row-major inside the computed rectangle).
template <typename XT>
__global__ __launch_bounds__(256) void k_proj(Dev D, const XT* __restrict__ xc, int C, int H,
                                              const float* __restrict__ Wx, const float* __restrict__ bias,
                                              float* __restrict__ Z) {
    const int lane = threadIdx.x & 63;
    const int64_t cell0 = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * 16;
    if (cell0 >= D.T) return;  // whole wave leaves together
    const int G = 5 * H;
    const int NT = 4 * G;
    float* Z1 = Z + z1_offset(D.T, H);

    // A operand: lane supplies x[cell0 + (lane % 16)][4*ks + lane / 16]
    const int64_t ca = cell0 + (lane & 15);
    int64_t xbase = -1;
    if (ca < D.T) {
        const int e = find_example(D.cell_off, D.n, ca);
        const int w = D.rect[4 * e + 3];
        const int64_t q = ca - D.cell_off[e];
        const int ly = (int)(q / w), lx = (int)(q % w);
        xbase = ((int64_t)(D.rect[4 * e] + ly) * D.Wc + D.rect[4 * e + 1] + lx) * C;
    }
    // output rows of this lane: cells cell0 + 4*(lane/16) + r, r = 0..3; their stash index per direction
    int64_t dst[4][4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int64_t c = cell0 + 4 * (lane >> 4) + r;
        if (c < D.T) {
            const int e = find_example(D.cell_off, D.n, c);
            const int h = D.rect[4 * e + 2], w = D.rect[4 * e + 3];
            const int64_t q = c - D.cell_off[e];
            const int ly = (int)(q / w), lx = (int)(q % w);
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                const int a = (d & 2) ? h - 1 - ly : ly;
                const int b = (d & 1) ? w - 1 - lx : lx;
                const int s = a + b;
                dst[r][d] = (int64_t)d * D.T + D.cell_off[e] + dg_start(h, w, s) + (a - dg_lo(h, w, s));
            }
        } else {
#pragma unroll
            for (int d = 0; d < 4; ++d) dst[r][d] = -1;
        }
    }
    const int ksteps = (C + 3) >> 2;
    for (int n0 = 0; n0 < NT; n0 += 16) {
        const int n = n0 + (lane & 15);
        const bool nok = n < NT;
        const int d = nok ? n / G : 0;
        const int gcol = nok ? n - d * G : 0;
        const int g = gcol / H, k = gcol - g * H;  // gate, hidden unit
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        for (int ks = 0; ks < ksteps; ++ks) {
            const int k = 4 * ks + (lane >> 4);
            const float av = (xbase >= 0 && k < C) ? to_f32<XT>(xc[xbase + k]) : 0.f;
            const float bv = (nok && k < C) ? Wx[((int64_t)d * C + k) * G + gcol] : 0.f;
            acc = __builtin_amdgcn_mfma_f32_16x16x4f32(av, bv, acc, 0, 0, 0);
        }
        if (nok) {
            const float bb = bias[d * G + gcol];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                // select without dynamic register indexing
                const int64_t t = d == 0 ? dst[r][0] : d == 1 ? dst[r][1] : d == 2 ? dst[r][2] : dst[r][3];
                if (t >= 0) {
                    if (g < 4) Z[(t * H + k) * 4 + g] = acc[r] + bb;
                    else Z1[t * H + k] = acc[r] + bb;
                }
            }
        }
    }
}

}  // namespace

hipError_t launch_projection(const Dev& D, const void* x_canvas, int dtype, int C, int H, const float* Wx,
                             const float* b, float* Z, hipStream_t st) {
    const int64_t waves = (D.T + 15) / 16;
    const unsigned blocks = (unsigned)((waves + 3) / 4);
    if (dtype == 0)
        launch(k_proj<float>, dim3(blocks), dim3(256), 0, st, D, (const float*)x_canvas, C, H, Wx, b, Z);
    else
        launch(k_proj<uint16_t>, dim3(blocks), dim3(256), 0, st, D, (const uint16_t*)x_canvas, C, H,
               Wx, b, Z);
    return hipGetLastError();
}

}  // namespace mdl
