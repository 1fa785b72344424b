// devmath.h — device helpers shared by the wavefront and gradient kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace mdl {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
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
// about 1 ulp each). sigmoid(z) = 1 / (1 + e^-z). tanh(x) = 2 / (1 + e^-2x) - 1 for
// |x| >= 1/8 (absolute error about 1e-7, relative below 1e-6 there; finite for any x),
// and below 1/8 its odd Taylor polynomial to x^7 (truncation below 2e-9 relative), so
// that tanh keeps its relative accuracy near 0 instead of losing it to cancellation.
// Both branches are computed and one is selected: no divergence.
__device__ inline float fexp(float x) { return __builtin_amdgcn_exp2f(x * 1.44269504088896341f); }
__device__ inline float frcp(float x) { return __builtin_amdgcn_rcpf(x); }
__device__ inline float sigm(float z) { return frcp(1.0f + fexp(-z)); }
// e^-2x as 2^(x (-2 log2 e)): -2 times the float log2 e is exact, and scaling by a power of two commutes with
// rounding, so this is bit for bit exp2((-2x) log2 e) at one multiply fewer.
constexpr float kM2L2E = -2.0f * 1.44269504088896341f;
__device__ inline float ftanh(float x) {
    const float big = __builtin_fmaf(2.0f, frcp(1.0f + __builtin_amdgcn_exp2f(x * kM2L2E)), -1.0f);
    const float x2 = x * x;
    const float p = __builtin_fmaf(x2, __builtin_fmaf(x2, -17.0f / 315.0f, 2.0f / 15.0f), -1.0f / 3.0f);
    const float small = __builtin_fmaf(x * x2, p, x);
    return fabsf(x) < 0.125f ? small : big;
}

// fp32 value -> f16 pair (hi, lo) with hi + lo equal to v to about 2^-22 relative,
// for |v| < 65504 and |v| above the f16 normal range's floor.
__device__ inline void split16(float v, _Float16& hi, _Float16& lo) {
    hi = (_Float16)v;
    lo = (_Float16)(v - (float)hi);
}

}  // namespace mdl
