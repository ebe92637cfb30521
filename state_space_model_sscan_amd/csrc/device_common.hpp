// device_common.hpp -- small device helpers shared by the libsscan kernels (gfx950).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sscan {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// bf16 <-> f32. Loads are exact; stores round to nearest even (NaN stays NaN):
// gfx950 converts in one instruction (v_cvt_pk_bf16_f32).
__device__ __forceinline__ float bf16_to_f32(uint16_t v) { return __uint_as_float((uint32_t)v << 16); }
__device__ __forceinline__ uint16_t f32_to_bf16(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }

template <typename T> struct Act;
template <> struct Act<float> {
  static __device__ __forceinline__ float ld(const float* p) { return *p; }
  static __device__ __forceinline__ void st(float* p, float v) { *p = v; }
};
template <> struct Act<uint16_t> {
  static __device__ __forceinline__ float ld(const uint16_t* p) { return bf16_to_f32(*p); }
  static __device__ __forceinline__ void st(uint16_t* p, float v) { *p = f32_to_bf16(v); }
};

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }
__device__ __forceinline__ float fast_rcp(float x) { return __builtin_amdgcn_rcpf(x); }

// softplus(v) = log(1 + e^v) = max(v, 0) + log1p(e^-|v|).
// log1p(e) for e in [0, 1] is log(u) with u = fl(1 + e), corrected by the
// rounding error of u: log(1 + e) = log(u) - ((u - 1) - e) / u to first order;
// (u - 1) - e is exact. softplus(-inf) = 0 exactly (a zero step).
__device__ __forceinline__ float softplus(float v) {
  const float e = fast_exp2(-fabsf(v) * kLog2e);
  const float u = 1.0f + e;
  const float corr = (u - 1.0f) - e;
  const float l = fast_log2(u) * kLn2 - corr * fast_rcp(u);
  return fmaxf(v, 0.0f) + l;
}

// softplus without the rounding correction of 1 + e. Its absolute error in dt is
// below 2^-24 (the rounding of 1 + e), which enters the scan only through
// dt * x * B and dt * A: negligible next to fp32 rounding of the state. Used in the
// hot loops; softplus() above where a step is computed once per call.
__device__ __forceinline__ float softplus_fast(float v) {
  const float e = fast_exp2(-fabsf(v) * kLog2e);
  return fmaf(fast_log2(1.0f + e), kLn2, fmaxf(v, 0.0f));
}

// Bijective map of a linear block index onto an order in which consecutive
// logical blocks are dispatched to the same XCD (the dispatcher places block i
// on XCD i % 8), so neighbours that share cache lines share an L2.
__device__ __forceinline__ int64_t xcd_local_order(int64_t lin, int64_t n) {
  const int64_t xcd = lin % 8, k = lin / 8, q = n / 8, r = n % 8;
  return xcd * q + (xcd < r ? xcd : r) + k;
}

// silu(z) = z / (1 + e^-z); z -> -inf gives -0, z -> +inf gives z.
__device__ __forceinline__ float silu(float z) { return z * fast_rcp(1.0f + fast_exp2(-z * kLog2e)); }

}  // namespace sscan
