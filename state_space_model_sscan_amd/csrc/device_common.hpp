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

// The same sum with the two stages over lane bits 3 and 2 done without selects.
// Their classes are whole DPP banks (lanes 4k..4k+3 of a row), so one output is
// two bank-masked DPP adds into the same register: the first writes the banks of
// class 0 (its kept token plus the partner's copy of it), the second those of
// class 1; a lane outside a mask keeps what it holds. row_ror:r gives lane l the
// value of lane (l - r) mod 16, so the partner n^8 is row_ror:8 for both classes,
// and n^4 is row_ror:12 for class 0 (banks 0, 2: lane n + 4) and row_ror:4 for
// class 1 (banks 1, 3: lane n - 4). The masks gate only the writes: a lane still
// reads its partner in the other bank. The compiler has no form for a masked float
// add, hence the asm; `s_nop 1` gives the two wait states a DPP read needs after a
// VALU write of its source, so nothing depends on what the compiler scheduled
// before a block. The blocks have no effect beyond their outputs (not volatile,
// so the compiler may schedule them among other work). EXEC must be full (every
// lane of the row takes part). The stages
// over bits 1 and 0 are the select form above. Per 16 tokens: 33 VALU instructions
// against 45.
__device__ __forceinline__ float row_transpose_sum_banked(const float (&p)[16], int n) {
  float q[8], r[4], u[2];
  asm(
      "s_nop 1\n\t"
      "v_add_f32_dpp %0, %8, %8 row_ror:8 row_mask:0xf bank_mask:0x3\n\t"
      "v_add_f32_dpp %0, %16, %16 row_ror:8 row_mask:0xf bank_mask:0xc\n\t"
      "v_add_f32_dpp %1, %9, %9 row_ror:8 row_mask:0xf bank_mask:0x3\n\t"
      "v_add_f32_dpp %1, %17, %17 row_ror:8 row_mask:0xf bank_mask:0xc\n\t"
      "v_add_f32_dpp %2, %10, %10 row_ror:8 row_mask:0xf bank_mask:0x3\n\t"
      "v_add_f32_dpp %2, %18, %18 row_ror:8 row_mask:0xf bank_mask:0xc\n\t"
      "v_add_f32_dpp %3, %11, %11 row_ror:8 row_mask:0xf bank_mask:0x3\n\t"
      "v_add_f32_dpp %3, %19, %19 row_ror:8 row_mask:0xf bank_mask:0xc\n\t"
      "v_add_f32_dpp %4, %12, %12 row_ror:8 row_mask:0xf bank_mask:0x3\n\t"
      "v_add_f32_dpp %4, %20, %20 row_ror:8 row_mask:0xf bank_mask:0xc\n\t"
      "v_add_f32_dpp %5, %13, %13 row_ror:8 row_mask:0xf bank_mask:0x3\n\t"
      "v_add_f32_dpp %5, %21, %21 row_ror:8 row_mask:0xf bank_mask:0xc\n\t"
      "v_add_f32_dpp %6, %14, %14 row_ror:8 row_mask:0xf bank_mask:0x3\n\t"
      "v_add_f32_dpp %6, %22, %22 row_ror:8 row_mask:0xf bank_mask:0xc\n\t"
      "v_add_f32_dpp %7, %15, %15 row_ror:8 row_mask:0xf bank_mask:0x3\n\t"
      "v_add_f32_dpp %7, %23, %23 row_ror:8 row_mask:0xf bank_mask:0xc"
      : "=&v"(q[0]), "=&v"(q[1]), "=&v"(q[2]), "=&v"(q[3]), "=&v"(q[4]), "=&v"(q[5]), "=&v"(q[6]), "=&v"(q[7])
      : "v"(p[0]), "v"(p[1]), "v"(p[2]), "v"(p[3]), "v"(p[4]), "v"(p[5]), "v"(p[6]), "v"(p[7]), "v"(p[8]),
        "v"(p[9]), "v"(p[10]), "v"(p[11]), "v"(p[12]), "v"(p[13]), "v"(p[14]), "v"(p[15]));
  asm(
      "s_nop 1\n\t"
      "v_add_f32_dpp %0, %4, %4 row_ror:12 row_mask:0xf bank_mask:0x5\n\t"
      "v_add_f32_dpp %0, %8, %8 row_ror:4 row_mask:0xf bank_mask:0xa\n\t"
      "v_add_f32_dpp %1, %5, %5 row_ror:12 row_mask:0xf bank_mask:0x5\n\t"
      "v_add_f32_dpp %1, %9, %9 row_ror:4 row_mask:0xf bank_mask:0xa\n\t"
      "v_add_f32_dpp %2, %6, %6 row_ror:12 row_mask:0xf bank_mask:0x5\n\t"
      "v_add_f32_dpp %2, %10, %10 row_ror:4 row_mask:0xf bank_mask:0xa\n\t"
      "v_add_f32_dpp %3, %7, %7 row_ror:12 row_mask:0xf bank_mask:0x5\n\t"
      "v_add_f32_dpp %3, %11, %11 row_ror:4 row_mask:0xf bank_mask:0xa"
      : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3])
      : "v"(q[0]), "v"(q[1]), "v"(q[2]), "v"(q[3]), "v"(q[4]), "v"(q[5]), "v"(q[6]), "v"(q[7]));
  const bool c1 = n & 2, c0 = n & 1;
#pragma unroll
  for (int i = 0; i < 2; ++i) u[i] = tr_stage<0x4E>(r[i], r[i + 2], c1);
  return tr_stage<0xB1>(u[0], u[1], c0);
}

}  // namespace sscan
