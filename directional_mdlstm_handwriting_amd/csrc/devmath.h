// devmath.h — device helpers shared by the wavefront and gradient kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace mdl {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

// Raw buffer loads/stores on a per-unit buffer descriptor. A lane with nothing
// to load or store passes an offset past the descriptor's range: the hardware
// returns 0 for the load and drops the store. Every lane then issues the same
// memory instructions with no branch around them, so the compiler can wait
// for one prefetch with vmcnt(N) while earlier stores stay in flight (loads
// and stores share one in-order counter on this architecture).
constexpr uint32_t kBufCfg = 0x00020000;  // dword 3 of a raw 32-bit buffer descriptor (gfx9 family)

__device__ inline __amdgpu_buffer_rsrc_t rsrc(const void* base, int64_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, (int)kBufCfg);
}
__device__ inline float bld(__amdgpu_buffer_rsrc_t r, int off) {
    return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}
__device__ inline void bst(float v, __amdgpu_buffer_rsrc_t r, int off) {
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, off, 0, 0);
}

// Gate nonlinearities on the hardware exp2 and reciprocal (v_exp_f32, v_rcp_f32,
// about 1 ulp each). sigmoid(z) = 1 / (1 + e^-z).
// tanh: for |x| >= 0.55, 1 - 2 / (e^{2|x|} + 1) with the sign of x; there e^{2|x|} >= 3, so the
// subtraction leaves a result of at least 0.5 and loses no bits. Below 0.55, the odd polynomial
// x + x^3 P(x^2), P of degree 4 with coefficients fitted to tanh on [0, 0.55] by least squares in the
// relative error (truncation below 1.1e-9). Evaluated in fp32 with exact exp2 and reciprocal, the two
// branches stay within 1.7 ulp of tanh for every x (0.7 ulp below 0.55). The form 2 / (1 + e^-2x) - 1
// used before cancelled between 1/8 and 0.55 (up to 13 ulp), and that error, carried by o tanh(c) and by
// 1 - tanh^2 into every gradient, was the largest part of the gap to a plain fp32 evaluation.
// Both branches are computed and one is selected: no divergence; finite for every finite x.
__device__ inline float fexp(float x) { return __builtin_amdgcn_exp2f(x * 1.44269504088896341f); }
__device__ inline float frcp(float x) { return __builtin_amdgcn_rcpf(x); }
__device__ inline float sigm(float z) { return frcp(1.0f + fexp(-z)); }
constexpr float k2L2E = 2.0f * 1.44269504088896341f;  // e^{2y} = 2^{y (2 log2 e)}
constexpr float kTc0 = -0.3333331865184439f, kTc1 = 0.1333261685730572f, kTc2 = -0.053855118770899185f,
                kTc3 = 0.021082054635114145f, kTc4 = -0.006287655483799332f;
__device__ inline float ftanh(float x) {
    const float ax = fabsf(x);
    const float big = __builtin_fmaf(-2.0f, frcp(__builtin_amdgcn_exp2f(ax * k2L2E) + 1.0f), 1.0f);
    const float x2 = x * x;
    float p = __builtin_fmaf(x2, kTc4, kTc3);
    p = __builtin_fmaf(x2, p, kTc2);
    p = __builtin_fmaf(x2, p, kTc1);
    p = __builtin_fmaf(x2, p, kTc0);
    const float small = __builtin_fmaf(x * x2, p, x);
    return ax < 0.55f ? small : __builtin_copysignf(big, x);
}

// The factors the reverse wavefront multiplies a cell's gradients by, from the cell's forward values (gates
// i, f_l, f_u, o, cell input g, tc = tanh c) and its predecessors' memory states c_l, c_u:
//   A = (g i(1-i), c_l f_l(1-f_l), c_u f_u(1-f_u), tc o(1-o)),  B = (i(1-g^2), o(1-tc^2), f_l, f_u)
// so that dc = dh B[1] + dc_in and da = (dc A[0], dc A[1], dc A[2], dh A[3], dc B[0]). The forward stashes
// (i, f_l, f_u, o) and (g, tc, c_l, c_u); this forms the factors from the two vectors.
__device__ inline void bwd_factors(float ig, float fl, float fu, float og, float gg, float cl, float cu, float tc,
                                   f32x4& A, f32x4& B) {
    A = f32x4{gg * (ig * (1.f - ig)), cl * (fl * (1.f - fl)), cu * (fu * (1.f - fu)), tc * (og * (1.f - og))};
    B = f32x4{ig * (1.f - gg * gg), og * (1.f - tc * tc), fl, fu};
}
__device__ inline void bwd_factors(f32x4 gates, f32x4 rest, f32x4& A, f32x4& B) {
    bwd_factors(gates[0], gates[1], gates[2], gates[3], rest[0], rest[2], rest[3], rest[1], A, B);
}

// fp32 value -> f16 pair (hi, lo) with hi + lo equal to v to about 2^-22 relative,
// for |v| < 65504 and |v| above the f16 normal range's floor.
__device__ inline void split16(float v, _Float16& hi, _Float16& lo) {
    hi = (_Float16)v;
    lo = (_Float16)(v - (float)hi);
}

}  // namespace mdl
