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

// softplus as above with the correction subtracted undivided: corr / u and corr
// differ by corr * e / u, below 2^-24 e, while log1p(e) >= e / 2, so the step
// keeps a relative error of a few ulp at every size (without the correction a
// step of 1e-4 would carry a relative error near 6e-4). Saves the reciprocal in
// the hot loops.
__device__ __forceinline__ float softplus_fast(float v) {
  const float e = fast_exp2(-fabsf(v) * kLog2e);
  const float u = 1.0f + e;
  const float corr = (u - 1.0f) - e;
  return fmaf(fast_log2(u), kLn2, fmaxf(v, 0.0f)) - corr;
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

// DPP helpers for the 16-lane rows of a wave (gfx950).
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// One exchange stage of the row transpose-reduce: tokens lo (class 0 keeps) and
// hi (class 1 keeps); the partner lane (CTRL) is in the other class.
template <int CTRL>
__device__ __forceinline__ float tr_stage(float lo, float hi, bool cls) {
  const float keep = cls ? hi : lo;
  const float send = cls ? lo : hi;
  return keep + dpp_f<CTRL>(send);
}

// p[t] holds this lane's term for token t of a 16-token group; returns, in lane n
// of each row, the sum of p[n] over the 16 lanes of the row. Stage partners:
// n^8 (row_ror:8), n^7 (row_half_mirror), n^2 and n^1 (quad_perm); the vectors
// 8, 7, 2, 1 span all 16 lanes, and the classes (bits 3, 2, 1, 0 of n) make the
// token kept at the end token n.
__device__ __forceinline__ float row_transpose_sum(const float (&p)[16], int n) {
  const bool c3 = n & 8, c2 = n & 4, c1 = n & 2, c0 = n & 1;
  float q[8], r[4], u[2];
#pragma unroll
  for (int i = 0; i < 8; ++i) q[i] = tr_stage<0x128>(p[i], p[i + 8], c3);
#pragma unroll
  for (int i = 0; i < 4; ++i) r[i] = tr_stage<0x141>(q[i], q[i + 4], c2);
#pragma unroll
  for (int i = 0; i < 2; ++i) u[i] = tr_stage<0x4E>(r[i], r[i + 2], c1);
  return tr_stage<0xB1>(u[0], u[1], c0);
}

}  // namespace sscan
