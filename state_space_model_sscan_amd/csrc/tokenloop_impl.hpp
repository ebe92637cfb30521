// tokenloop_impl.hpp -- token-loop selective scan kernels for gfx950: Mamba-1, and
// Mamba-2 SSD as its special case with one decay per head.
//
// The recurrence ("Mamba", nnterp guide, opening paragraph and section "The
// values"; "Mamba", tokentrails lineage, section "Code"): per channel c and
// state entry n,
//     dt  = softplus(dt_raw + dt_bias[c])
//     h_n = exp(dt * A[c, n]) * h_n + dt * B_n * x,     A = -exp(A_log)
//     y   = sum_n C_n h_n + D[c] * x,  then y * silu(z) when a gate is given.
// "Falcon-Mamba" (section "Where the norms sit"): optional weightless RMS norm
// of every [state_dim] vector of B and C before the scan.
//
// SSD mode ("Mamba-2", section "The mixer's values"): channel ch = h*P + p of
// head h holds the state row [p, :]; per head and token one step
// dt = softplus(dt_raw[b,t,h] + dt_bias[h]) and one decay exp(dt * A_h),
// A_h = -exp(A_log[h]), shared by every p and n; D per head. The stored state
// [b, H, P, N] is [b, channels, N] with channels = H*P.
//
// Mapping, up to 32 states (tokenloop_scan_kernel): one lane per channel, its
// state_dim entries in registers; one wave (64 lanes) per block of 64 channels
// of one batch row. B and C of a token are shared by every channel of the
// group, so the wave stages them (fp32, normed) in LDS once per tile of tokens
// and every lane reads them by broadcast. From 33 states up
// (tokenloop_group_kernel, below): 16 lanes per channel. The one-token decode
// step (tokenloop_step_kernel) uses 4 or 16 lanes per channel.
// exp(dt*A) is computed as exp2(dt * A*log2(e)) with A*log2(e) kept per lane.
//
// Sequence parallelism: the tokens of a batch row are cut into `nslices`
// slices. Pass 1 scans every slice but the last from a zero state and stores
// its end state and the sum of its steps; pass 2 starts slice s from
//     h = decay(slice j) * h + end_state(slice j),  j = 0 .. s-1,
// where the decay over slice j is exp(A * sum of dt over j), and scans it again,
// writing y, the optional per-token states and, for the last slice, the final
// state. Both passes restate the recurrence exactly; only rounding differs.
#pragma once
#include <type_traits>

#include "device_common.hpp"
#include "launch.hpp"

namespace sscan {

struct TLK {
  const void* x;
  const void* dt;
  const float* dt_bias;
  const float* A_log;
  const void* B;
  const void* C;
  const float* D;
  const void* z;
  const float* h0;
  void* y;
  float* h_out;
  float* states;
  float* ws_h;    // [batch, nslices, Dc, N]
  float* ws_sdt;  // [batch, nslices, Dc]
  int64_t L, Dc;
  int N, G, nslices, slice_len;
  int64_t per_group;  // channels per B/C group
  float bc_eps;
  int64_t H, P;       // SSD mode: heads and head_dim (Dc = H * P)
};

// Tokens of B/C staged per LDS fill (at most the wave width, 64).
template <int NP> constexpr int tile_for() { return NP <= 32 ? 64 : (NP <= 64 ? 32 : 16); }

template <typename T, int NP, int TILE>
__device__ __forceinline__ void stage_bc(const TLK& k, int64_t row_tok, int g, float (*sB)[NP],
                                         float (*sC)[NP], int slot, bool want_c) {
  const T* Bp = (const T*)k.B + (row_tok * k.G + g) * k.N;
  const T* Cp = (const T*)k.C + (row_tok * k.G + g) * k.N;
  float ssb = 0.0f, ssc = 0.0f;
  for (int n = 0; n < NP; ++n) {
    const float bv = n < k.N ? Act<T>::ld(Bp + n) : 0.0f;
    const float cv = (want_c && n < k.N) ? Act<T>::ld(Cp + n) : 0.0f;
    sB[slot][n] = bv;
    if (want_c) sC[slot][n] = cv;
    ssb = fmaf(bv, bv, ssb);
    ssc = fmaf(cv, cv, ssc);
  }
  if (k.bc_eps > 0.0f) {
    const float ib = 1.0f / sqrtf(ssb / (float)k.N + k.bc_eps);
    const float ic = 1.0f / sqrtf(ssc / (float)k.N + k.bc_eps);
    for (int n = 0; n < NP; ++n) {
      sB[slot][n] *= ib;
      if (want_c) sC[slot][n] *= ic;
    }
  }
}

template <typename T, int NP, bool SSD, bool GATE, bool STATES, bool PASS1>
__global__ __launch_bounds__(64) void tokenloop_scan_kernel(TLK k) {
  constexpr int TILE = tile_for<NP>();
  __shared__ float sB[TILE][NP];
  __shared__ float sC[TILE][NP];
  const int lane = threadIdx.x;
  const int64_t c0 = (int64_t)blockIdx.x * 64;
  const int64_t c = c0 + lane;
  const bool active = c < k.Dc;
  const int64_t cc = active ? c : k.Dc - 1;
  const int s = blockIdx.y;
  const int64_t b = blockIdx.z;
  const int64_t t_begin = (int64_t)s * k.slice_len;
  const int64_t t_end = min(k.L, t_begin + (int64_t)k.slice_len);
  const int g = (int)(c0 / k.per_group);  // the host guarantees one group per wave
  const int64_t hd = SSD ? cc / k.P : cc;  // parameter index: head or channel

  float A2[SSD ? 1 : NP], h[NP];
  if (SSD) {
    A2[0] = -expf(k.A_log[hd]) * kLog2e;
  } else {
#pragma unroll
    for (int n = 0; n < NP; ++n) A2[SSD ? 0 : n] = n < k.N ? -expf(k.A_log[cc * k.N + n]) * kLog2e : 0.0f;
  }
#pragma unroll
  for (int n = 0; n < NP; ++n) h[n] = (!PASS1 && k.h0 && n < k.N) ? k.h0[(b * k.Dc + cc) * k.N + n] : 0.0f;
  if (!PASS1) {
    for (int j = 0; j < s; ++j) {
      const int64_t base = (b * k.nslices + j) * k.Dc + cc;
      const float sdt = k.ws_sdt[base];
      const float dec0 = SSD ? fast_exp2(A2[0] * sdt) : 0.0f;
#pragma unroll
      for (int n = 0; n < NP; ++n)
        if (n < k.N) h[n] = fmaf(SSD ? dec0 : fast_exp2(A2[SSD ? 0 : n] * sdt), h[n], k.ws_h[base * k.N + n]);
    }
  }

  const float bias = k.dt_bias[hd];
  const float Dv = PASS1 ? 0.0f : k.D[hd];
  const T* xp = (const T*)k.x;
  const T* dp = (const T*)k.dt;
  const T* zp = (const T*)k.z;
  T* yp = (T*)k.y;
  const int64_t dt_stride = SSD ? k.H : k.Dc;
  float sdt = 0.0f;

  for (int64_t t0 = t_begin; t0 < t_end; t0 += TILE) {
    const int nt = (int)min((int64_t)TILE, t_end - t0);
    __syncthreads();
    if (lane < nt) stage_bc<T, NP, TILE>(k, b * k.L + t0 + lane, g, sB, sC, lane, !PASS1);
    __syncthreads();
    for (int i = 0; i < nt; ++i) {
      const int64_t row = b * k.L + t0 + i;
      const int64_t idx = row * k.Dc + cc;
      const float xv = Act<T>::ld(xp + idx);
      const float dtv = softplus(Act<T>::ld(dp + row * dt_stride + hd) + bias);
      const float dtx = dtv * xv;
      const float dec0 = SSD ? fast_exp2(dtv * A2[0]) : 0.0f;
      if (PASS1) {
        sdt += dtv;
#pragma unroll
        for (int n = 0; n < NP; ++n)
          h[n] = fmaf(SSD ? dec0 : fast_exp2(dtv * A2[SSD ? 0 : n]), h[n], dtx * sB[i][n]);
      } else {
        float yv = Dv * xv;
#pragma unroll
        for (int n = 0; n < NP; ++n) {
          h[n] = fmaf(SSD ? dec0 : fast_exp2(dtv * A2[SSD ? 0 : n]), h[n], dtx * sB[i][n]);
          yv = fmaf(sC[i][n], h[n], yv);
        }
        if (STATES && active) {
          if constexpr (NP % 4 == 0) {
            if (k.N == NP) {  // whole 16-byte pieces: rows of N floats are 16-byte aligned
              typedef float f32x4_t __attribute__((ext_vector_type(4)));
#pragma unroll
              for (int n = 0; n < NP; n += 4)
                *(f32x4_t*)(k.states + idx * NP + n) = f32x4_t{h[n], h[n + 1], h[n + 2], h[n + 3]};
            } else {
#pragma unroll
              for (int n = 0; n < NP; ++n)
                if (n < k.N) k.states[idx * k.N + n] = h[n];
            }
          } else {
#pragma unroll
            for (int n = 0; n < NP; ++n)
              if (n < k.N) k.states[idx * k.N + n] = h[n];
          }
        }
        if (GATE) yv *= silu(Act<T>::ld(zp + idx));
        if (active) Act<T>::st(yp + idx, yv);
      }
    }
  }

  if (PASS1) {
    if (active) {
      const int64_t base = (b * k.nslices + s) * k.Dc + c;
#pragma unroll
      for (int n = 0; n < NP; ++n)
        if (n < k.N) k.ws_h[base * k.N + n] = h[n];
      k.ws_sdt[base] = sdt;
    }
  } else if (s == k.nslices - 1 && active) {
#pragma unroll
    for (int n = 0; n < NP; ++n)
      if (n < k.N) k.h_out[(b * k.Dc + c) * k.N + n] = h[n];
  }
}

// Contiguous loads of NQ elements into fp32 registers in 16-byte pieces (or the
// whole run when it is shorter); the caller guarantees the alignment.
template <int NQ>
__device__ __forceinline__ void ld_run(const float* p, float (&o)[NQ]) {
  typedef float f32x4_t __attribute__((ext_vector_type(4)));
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  if constexpr (NQ % 4 == 0) {
#pragma unroll
    for (int i = 0; i < NQ; i += 4) {
      const f32x4_t v = *(const f32x4_t*)(p + i);
      o[i] = v[0]; o[i + 1] = v[1]; o[i + 2] = v[2]; o[i + 3] = v[3];
    }
  } else {
    static_assert(NQ == 2, "runs of 2 or a multiple of 4");
    const f32x2_t v = *(const f32x2_t*)p;
    o[0] = v[0]; o[1] = v[1];
  }
}
template <int NQ>
__device__ __forceinline__ void ld_run(const uint16_t* p, float (&o)[NQ]) {
  typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
  typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
  uint32_t w[NQ / 2];
  if constexpr (NQ % 8 == 0) {
#pragma unroll
    for (int i = 0; i < NQ / 2; i += 4) {
      const u32x4_t v = *(const u32x4_t*)(p + 2 * i);
      w[i] = v[0]; w[i + 1] = v[1]; w[i + 2] = v[2]; w[i + 3] = v[3];
    }
  } else if constexpr (NQ == 4) {
    const u32x2_t v = *(const u32x2_t*)p;
    w[0] = v[0]; w[1] = v[1];
  } else {
    static_assert(NQ == 2, "runs of 2, 4 or a multiple of 8");
    w[0] = *(const uint32_t*)p;
  }
#pragma unroll
  for (int i = 0; i < NQ / 2; ++i) {
    o[2 * i] = __uint_as_float(w[i] << 16);
    o[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}
template <int NQ>
__device__ __forceinline__ void st_run(float* p, const float (&v)[NQ]) {
  typedef float f32x4_t __attribute__((ext_vector_type(4)));
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  if constexpr (NQ % 4 == 0) {
#pragma unroll
    for (int i = 0; i < NQ; i += 4) *(f32x4_t*)(p + i) = f32x4_t{v[i], v[i + 1], v[i + 2], v[i + 3]};
  } else {
    *(f32x2_t*)p = f32x2_t{v[0], v[1]};
  }
}

// Lanes per channel of the one-token step: 4 below 64 state entries, else 16.
template <int NP>
constexpr int step_lanes() { return NP >= 64 ? 16 : 4; }

// Entry i of lane q. With 4 lanes a lane holds the contiguous quarter
// [q NQ, q NQ + NQ); with 16 lanes it holds 4-entry pieces at 64 c + 4 q, so
// that the 16 lanes of a channel read 256 contiguous bytes of fp32 state per
// load instruction.
template <int NP>
__device__ __forceinline__ int step_entry(int q, int i) {
  constexpr int K = step_lanes<NP>(), NQ = NP / K;
  return K == 4 ? q * NQ + i : 64 * (i >> 2) + 4 * q + (i & 3);
}

// NQ entries of lane q from a row whose every entry is present (N == NP).
template <int NP, typename E>
__device__ __forceinline__ void step_ld(const E* row, int q, float (&o)[NP / step_lanes<NP>()]) {
  constexpr int K = step_lanes<NP>(), NQ = NP / K;
  if constexpr (K == 4) {
    ld_run<NQ>(row + q * NQ, o);
  } else {
#pragma unroll
    for (int c = 0; c < NQ / 4; ++c) {
      float t[4];
      ld_run<4>(row + 64 * c + 4 * q, t);
#pragma unroll
      for (int i = 0; i < 4; ++i) o[4 * c + i] = t[i];
    }
  }
}

template <int NP>
__device__ __forceinline__ void step_st(float* row, int q, const float (&v)[NP / step_lanes<NP>()]) {
  constexpr int K = step_lanes<NP>(), NQ = NP / K;
  if constexpr (K == 4) {
    st_run<NQ>(row + q * NQ, v);
  } else {
#pragma unroll
    for (int c = 0; c < NQ / 4; ++c) {
      const float t[4] = {v[4 * c], v[4 * c + 1], v[4 * c + 2], v[4 * c + 3]};
      st_run<4>(row + 64 * c + 4 * q, t);
    }
  }
}

// Sum over the K lanes of a channel (xor butterfly inside the lane group).
// (K = 16: the lane group is one DPP row of the wave; after the quad sums, rotating the
// row by 4 and then by 8 lanes adds the other three quads, so every lane of the row ends
// with the row's sum, with no round trip through the LDS crossbar)
template <int K>
__device__ __forceinline__ float step_sum(float v) {
  static_assert(K == 4 || K == 16, "lane groups of 4 or 16");
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false));  // quad_perm 1,0,3,2
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, false));  // quad_perm 2,3,0,1
  if constexpr (K == 16) {
    v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x124, 0xF, 0xF, false));  // row_ror:4
    v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x128, 0xF, 0xF, false));  // row_ror:8
  }
  return v;
}

// One token per call: K lanes per channel (step_lanes), each holding NP / K of
// its state_dim entries (step_entry), so that a channel's state, A_log, B and C
// move as whole pieces of 16 bytes or more. The state is read, updated, then y
// is read from the updated state ("Mamba", section "The state"). The partial
// read-outs are summed over the lane group, and its lane 0 stores y. When
// state_dim is below the padded NP, the entries are read one by one with a
// bound check.
template <typename T, int NP, bool SSD, bool GATE>
__global__ __launch_bounds__(256) void tokenloop_step_kernel(TLK k) {
  constexpr int K = step_lanes<NP>();
  constexpr int NQ = NP / K;  // entries per lane
  const int64_t gl = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int q = (int)(gl % K);
  const int64_t c = gl / K;
  const int64_t b = blockIdx.y;
  const bool active = c < k.Dc;
  const int64_t cc = active ? c : k.Dc - 1;  // inactive lanes compute on a valid channel, store nothing
  const int g = (int)(cc / k.per_group);
  const int64_t hd = SSD ? cc / k.P : cc;
  const int64_t sidx = (b * k.Dc + cc) * k.N;
  const T* Bp = (const T*)k.B + (b * k.G + g) * k.N;
  const T* Cp = (const T*)k.C + (b * k.G + g) * k.N;
  const bool full = k.N == NP;  // every entry present: rows are NP-aligned runs
  float bv[NQ], cv[NQ], hv[NQ];
  if (full) {
    step_ld<NP>(Bp, q, bv);
    step_ld<NP>(Cp, q, cv);
    step_ld<NP>(k.h0 + sidx, q, hv);
  } else {
#pragma unroll
    for (int i = 0; i < NQ; ++i) {
      const int n = step_entry<NP>(q, i);
      bv[i] = n < k.N ? Act<T>::ld(Bp + n) : 0.0f;
      cv[i] = n < k.N ? Act<T>::ld(Cp + n) : 0.0f;
      hv[i] = n < k.N ? k.h0[sidx + n] : 0.0f;
    }
  }
  float ib = 1.0f, ic = 1.0f;
  if (k.bc_eps > 0.0f) {
    float sb = 0.0f, sc = 0.0f;
#pragma unroll
    for (int i = 0; i < NQ; ++i) {
      sb = fmaf(bv[i], bv[i], sb);
      sc = fmaf(cv[i], cv[i], sc);
    }
    sb = step_sum<K>(sb);
    sc = step_sum<K>(sc);
    ib = 1.0f / sqrtf(sb / (float)k.N + k.bc_eps);
    ic = 1.0f / sqrtf(sc / (float)k.N + k.bc_eps);
  }
  float av[NQ];  // A_log of the entries (Mamba-1)
  if constexpr (!SSD) {
    if (full) {
      step_ld<NP>(k.A_log + cc * k.N, q, av);
    } else {
#pragma unroll
      for (int i = 0; i < NQ; ++i) {
        const int n = step_entry<NP>(q, i);
        av[i] = n < k.N ? k.A_log[cc * k.N + n] : 0.0f;
      }
    }
  }
  const int64_t idx = b * k.Dc + cc;  // seqlen 1
  const float xv = Act<T>::ld((const T*)k.x + idx);
  const float dtv = softplus(Act<T>::ld((const T*)k.dt + b * (SSD ? k.H : k.Dc) + hd) + k.dt_bias[hd]);
  const float dtx = dtv * xv;
  const float dec0 = SSD ? fast_exp2(dtv * (-fast_exp2(k.A_log[hd] * kLog2e) * kLog2e)) : 0.0f;
  float acc = 0.0f;
  float h[NQ];
#pragma unroll
  for (int i = 0; i < NQ; ++i) {
    // padded entries (n >= N) hold zeros in B, C and the state, and stay zero
    const float dec = SSD ? dec0 : fast_exp2(dtv * (-fast_exp2(av[i] * kLog2e) * kLog2e));
    h[i] = fmaf(dec, hv[i], dtx * (bv[i] * ib));
    acc = fmaf(cv[i] * ic, h[i], acc);
  }
  acc = step_sum<K>(acc);
  float yv = acc + k.D[hd] * xv;
  if (GATE) yv *= silu(Act<T>::ld((const T*)k.z + idx));
  if (active) {
    if (q == 0) Act<T>::st((T*)k.y + idx, yv);
    if (full) {
      step_st<NP>(k.h_out + sidx, q, h);
    } else {
#pragma unroll
      for (int i = 0; i < NQ; ++i) {
        const int n = step_entry<NP>(q, i);
        if (n < k.N) k.h_out[sidx + n] = h[i];
      }
    }
  }
}

// Token loop for wide states (padded state_dim 64, 128 or 256): 16 lanes per channel,
// each holding the entries step_entry() gives it, 16 channels per 256-thread
// block. One lane per channel would leave a 128-entry state in 256 registers,
// a few waves on the chip and, with per-token states, 4-byte stores 512 bytes
// apart; here the 16 lanes of a channel store 256 contiguous bytes per
// instruction. Per tile of tokens the block stages B and C (fp32, normed when
// asked) and, per channel, x, z and the step dt = softplus(dt_raw + dt_bias) in
// LDS; the read-out is a sum over the 16 lanes. Slices and the carry between
// them work as in tokenloop_scan_kernel, with the same workspace layout.
// Tokens per staging of the group kernel: 32, or 16 for 256 states (B and C of a
// tile then take 32 KiB of LDS).
template <int NP> constexpr int group_tile() { return NP >= 256 ? 16 : 32; }

template <typename T, int NP, bool SSD, bool GATE, bool STATES, bool PASS1>
__global__ __launch_bounds__(256) void tokenloop_group_kernel(TLK k) {
  constexpr int K = step_lanes<NP>();
  static_assert(K == 16, "wide states only");
  constexpr int NQ = NP / K;
  constexpr int TILE = group_tile<NP>();
  constexpr int CPB = 256 / K;  // channels per block
  __shared__ __attribute__((aligned(16))) float sB[TILE][NP];
  __shared__ __attribute__((aligned(16))) float sC[TILE][NP];
  __shared__ float sX[TILE][CPB], sDT[TILE][CPB], sZ[TILE][CPB];
  __shared__ float sNB[TILE], sNC[TILE];
  const int tid = threadIdx.x;
  const int q = tid % K, cl = tid / K;
  const int64_t c0 = (int64_t)blockIdx.x * CPB;
  const int64_t c = c0 + cl;
  const bool active = c < k.Dc;
  const int64_t cc = active ? c : k.Dc - 1;
  const int s = blockIdx.y;
  const int64_t b = blockIdx.z;
  const int64_t t_begin = (int64_t)s * k.slice_len;
  const int64_t t_end = min(k.L, t_begin + (int64_t)k.slice_len);
  const int g = (int)(c0 / k.per_group);  // the host guarantees one group per block
  const int64_t hd = SSD ? cc / k.P : cc;
  const bool full = k.N == NP;

  float A2[SSD ? 1 : NQ], h[NQ];
  if constexpr (SSD) {
    A2[0] = -expf(k.A_log[hd]) * kLog2e;
  } else {
#pragma unroll
    for (int e = 0; e < NQ; ++e) {
      const int n = step_entry<NP>(q, e);
      A2[e] = n < k.N ? -expf(k.A_log[cc * k.N + n]) * kLog2e : 0.0f;
    }
  }
  const int64_t sbase = (b * k.Dc + cc) * k.N;
#pragma unroll
  for (int e = 0; e < NQ; ++e) h[e] = 0.0f;
  if (!PASS1 && k.h0) {
    if (full) {
      step_ld<NP>(k.h0 + sbase, q, h);
    } else {
#pragma unroll
      for (int e = 0; e < NQ; ++e) {
        const int n = step_entry<NP>(q, e);
        h[e] = n < k.N ? k.h0[sbase + n] : 0.0f;
      }
    }
  }
  if (!PASS1) {
    for (int j = 0; j < s; ++j) {
      const int64_t base = (b * k.nslices + j) * k.Dc + cc;
      const float sdt = k.ws_sdt[base];
      float wh[NQ];
      if (full) {
        step_ld<NP>(k.ws_h + base * NP, q, wh);
      } else {
#pragma unroll
        for (int e = 0; e < NQ; ++e) {
          const int n = step_entry<NP>(q, e);
          wh[e] = n < k.N ? k.ws_h[base * k.N + n] : 0.0f;
        }
      }
      const float dec0 = SSD ? fast_exp2(A2[0] * sdt) : 0.0f;
#pragma unroll
      for (int e = 0; e < NQ; ++e) h[e] = fmaf(SSD ? dec0 : fast_exp2(A2[SSD ? 0 : e] * sdt), h[e], wh[e]);
    }
  }

  const float Dv = PASS1 ? 0.0f : k.D[hd];
  const T* xp = (const T*)k.x;
  const T* dp = (const T*)k.dt;
  const T* zp = (const T*)k.z;
  T* yp = (T*)k.y;
  const int64_t dt_stride = SSD ? k.H : k.Dc;
  float sdt = 0.0f;

  for (int64_t t0 = t_begin; t0 < t_end; t0 += TILE) {
    const int nt = (int)min((int64_t)TILE, t_end - t0);
    __syncthreads();  // the previous tile is consumed
    for (int e = tid; e < TILE * NP; e += 256) {
      const int t = e / NP, n = e % NP;
      const int64_t row = b * k.L + t0 + t;
      const bool ok = t < nt && n < k.N;
      sB[t][n] = ok ? Act<T>::ld((const T*)k.B + (row * k.G + g) * k.N + n) : 0.0f;
      if (!PASS1) sC[t][n] = ok ? Act<T>::ld((const T*)k.C + (row * k.G + g) * k.N + n) : 0.0f;
    }
    for (int e = tid; e < TILE * CPB; e += 256) {
      const int t = e / CPB, ch = e % CPB;
      const int64_t cx = min(c0 + ch, k.Dc - 1);
      const int64_t row = b * k.L + t0 + t;
      const int64_t hx = SSD ? cx / k.P : cx;
      const bool ok = t < nt;
      sX[t][ch] = ok ? Act<T>::ld(xp + row * k.Dc + cx) : 0.0f;
      sDT[t][ch] = ok ? softplus(Act<T>::ld(dp + row * dt_stride + hx) + k.dt_bias[hx]) : 0.0f;
      if (GATE && !PASS1) sZ[t][ch] = ok ? Act<T>::ld(zp + row * k.Dc + cx) : 0.0f;
    }
    __syncthreads();
    if (k.bc_eps > 0.0f) {
      if (tid < TILE) {
        float sb = 0.0f, sc = 0.0f;
        for (int n = 0; n < NP; ++n) {
          sb = fmaf(sB[tid][n], sB[tid][n], sb);
          if (!PASS1) sc = fmaf(sC[tid][n], sC[tid][n], sc);
        }
        sNB[tid] = 1.0f / sqrtf(sb / (float)k.N + k.bc_eps);
        sNC[tid] = 1.0f / sqrtf(sc / (float)k.N + k.bc_eps);
      }
      __syncthreads();
      // the normed B and C in place, once per tile (the per-token loop then needs no
      // scaling; B * ib is formed first either way, so the rounding is the same)
      for (int e = tid; e < TILE * NP; e += 256) {
        const int t = e / NP, n = e % NP;
        sB[t][n] *= sNB[t];
        if (!PASS1) sC[t][n] *= sNC[t];
      }
      __syncthreads();
    }
    if (PASS1) {
      auto pass1_step = [&](int i) {
        const float dtv = sDT[i][cl];
        const float dtx = dtv * sX[i][cl];
        const float dec0 = SSD ? fast_exp2(dtv * A2[0]) : 0.0f;
        float bv[NQ];
        step_ld<NP>(&sB[i][0], q, bv);
        sdt += dtv;
#pragma unroll
        for (int e = 0; e < NQ; ++e) h[e] = fmaf(SSD ? dec0 : fast_exp2(dtv * A2[SSD ? 0 : e]), h[e], dtx * bv[e]);
      };
      // four tokens per iteration with no test between them (the LDS reads of the
      // four overlap), then the rest one by one
      int i = 0;
      for (; i + 4 <= nt; i += 4) {
#pragma unroll
        for (int j = 0; j < 4; ++j) pass1_step(i + j);
      }
      for (; i < nt; ++i) pass1_step(i);
    } else {
      // 16 tokens at a time: each lane keeps its partial read-out of every token,
      // then a transpose-reduce over the channel's 16 lanes (one DPP row) leaves
      // token i0 + q's sum in lane q, which finishes and stores that token's y.
      // A whole group runs without a test per token: with one, every token's state
      // update is a branch of its own and the compiler copies the state between
      // registers at each join (8 moves per token at 8 entries per lane).
      auto group = [&](int i0, auto tail) {
        constexpr bool TL = decltype(tail)::value;
        float p[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int i = i0 + j;
          p[j] = 0.0f;
          if (!TL || i < nt) {
            const float dtv = sDT[i][cl];
            const float dtx = dtv * sX[i][cl];
            const float dec0 = SSD ? fast_exp2(dtv * A2[0]) : 0.0f;
            float bv[NQ], cv[NQ];
            step_ld<NP>(&sB[i][0], q, bv);
            step_ld<NP>(&sC[i][0], q, cv);
            float acc = 0.0f;
#pragma unroll
            for (int e = 0; e < NQ; ++e) {
              h[e] = fmaf(SSD ? dec0 : fast_exp2(dtv * A2[SSD ? 0 : e]), h[e], dtx * bv[e]);
              acc = fmaf(cv[e], h[e], acc);
            }
            p[j] = acc;
            if (STATES && active) {
              const int64_t idx = (b * k.L + t0 + i) * k.Dc + cc;
              if (full) {  // non-temporal: the per-token states are not read again here
                typedef float f32x4_t __attribute__((ext_vector_type(4)));
#pragma unroll
                for (int c4 = 0; c4 < NQ / 4; ++c4)
                  __builtin_nontemporal_store(f32x4_t{h[4 * c4], h[4 * c4 + 1], h[4 * c4 + 2], h[4 * c4 + 3]},
                                              (f32x4_t*)(k.states + idx * NP + 64 * c4 + 4 * q));
              } else {
#pragma unroll
                for (int e = 0; e < NQ; ++e) {
                  const int n = step_entry<NP>(q, e);
                  if (n < k.N) k.states[idx * k.N + n] = h[e];
                }
              }
            }
          }
        }
        const float tot = row_transpose_sum(p, q);
        const int i = i0 + q;
        if (i < nt && active) {
          float yv = tot + Dv * sX[i][cl];
          if (GATE) yv *= silu(sZ[i][cl]);
          Act<T>::st(yp + (b * k.L + t0 + i) * k.Dc + cc, yv);
        }
      };
      for (int i0 = 0; i0 < nt; i0 += 16) {
        // (with per-token states the tested form stays: untested, the compiler keeps
        // all 16 tokens' states live for their stores, 322 registers against 90)
        if (!STATES && i0 + 16 <= nt) group(i0, std::false_type{});
        else group(i0, std::true_type{});
      }
    }
  }

  if (PASS1) {
    if (active) {
      const int64_t base = (b * k.nslices + s) * k.Dc + c;
      if (full) {
        step_st<NP>(k.ws_h + base * NP, q, h);
      } else {
#pragma unroll
        for (int e = 0; e < NQ; ++e) {
          const int n = step_entry<NP>(q, e);
          if (n < k.N) k.ws_h[base * k.N + n] = h[e];
        }
      }
      if (q == 0) k.ws_sdt[base] = sdt;
    }
  } else if (s == k.nslices - 1 && active) {
    if (full) {
      step_st<NP>(k.h_out + (b * k.Dc + c) * NP, q, h);
    } else {
#pragma unroll
      for (int e = 0; e < NQ; ++e) {
        const int n = step_entry<NP>(q, e);
        if (n < k.N) k.h_out[(b * k.Dc + c) * k.N + n] = h[e];
      }
    }
  }
}

static int padded_n(int64_t N) {
  return N <= 8 ? 8 : N <= 16 ? 16 : N <= 32 ? 32 : N <= 64 ? 64 : N <= 128 ? 128 : 256;
}

template <typename T, int NP, bool SSD>
static void launch_scan(const TLK& k, int64_t batch, bool gate, bool states, hipStream_t s) {
  if constexpr (NP >= 64) {  // wide states: 16 lanes per channel
    const dim3 blk(256);
    const int64_t cb = (k.Dc + 15) / 16;
    if (k.nslices > 1) {
      const dim3 grid1((unsigned)cb, (unsigned)(k.nslices - 1), (unsigned)batch);
      hipLaunchKernelGGL((tokenloop_group_kernel<T, NP, SSD, false, false, true>), grid1, blk, 0, s, k);
    }
    const dim3 grid((unsigned)cb, (unsigned)k.nslices, (unsigned)batch);
    if (gate && states)
      hipLaunchKernelGGL((tokenloop_group_kernel<T, NP, SSD, true, true, false>), grid, blk, 0, s, k);
    else if (gate)
      hipLaunchKernelGGL((tokenloop_group_kernel<T, NP, SSD, true, false, false>), grid, blk, 0, s, k);
    else if (states)
      hipLaunchKernelGGL((tokenloop_group_kernel<T, NP, SSD, false, true, false>), grid, blk, 0, s, k);
    else
      hipLaunchKernelGGL((tokenloop_group_kernel<T, NP, SSD, false, false, false>), grid, blk, 0, s, k);
  } else {  // one lane per channel
    const dim3 blk(64);
    const int64_t cb = (k.Dc + 63) / 64;
    if (k.nslices > 1) {
      const dim3 grid1((unsigned)cb, (unsigned)(k.nslices - 1), (unsigned)batch);
      hipLaunchKernelGGL((tokenloop_scan_kernel<T, NP, SSD, false, false, true>), grid1, blk, 0, s, k);
    }
    const dim3 grid((unsigned)cb, (unsigned)k.nslices, (unsigned)batch);
    if (gate && states)
      hipLaunchKernelGGL((tokenloop_scan_kernel<T, NP, SSD, true, true, false>), grid, blk, 0, s, k);
    else if (gate)
      hipLaunchKernelGGL((tokenloop_scan_kernel<T, NP, SSD, true, false, false>), grid, blk, 0, s, k);
    else if (states)
      hipLaunchKernelGGL((tokenloop_scan_kernel<T, NP, SSD, false, true, false>), grid, blk, 0, s, k);
    else
      hipLaunchKernelGGL((tokenloop_scan_kernel<T, NP, SSD, false, false, false>), grid, blk, 0, s, k);
  }
}

template <typename T, bool SSD>
void dispatch_scan(const TLK& k, int64_t batch, bool gate, bool states, hipStream_t s) {
  switch (padded_n(k.N)) {
    case 8: launch_scan<T, 8, SSD>(k, batch, gate, states, s); break;
    case 16: launch_scan<T, 16, SSD>(k, batch, gate, states, s); break;
    case 32: launch_scan<T, 32, SSD>(k, batch, gate, states, s); break;
    case 64: launch_scan<T, 64, SSD>(k, batch, gate, states, s); break;
    case 128: launch_scan<T, 128, SSD>(k, batch, gate, states, s); break;
    default:  // 129 to 256 states: Mamba-1 only (the host refuses wider SSD states)
      if constexpr (!SSD) launch_scan<T, 256, SSD>(k, batch, gate, states, s);
      break;
  }
}

// Pass 1 only: slice end states and step sums into the workspace.
template <typename T, bool SSD>
void dispatch_pass1(const TLK& k, int64_t batch, hipStream_t s) {
  const dim3 grid1((unsigned)((k.Dc + 63) / 64), (unsigned)(k.nslices - 1), (unsigned)batch), blk(64);
#define SSCAN_P1(NP) hipLaunchKernelGGL((tokenloop_scan_kernel<T, NP, SSD, false, false, true>), grid1, blk, 0, s, k);
  switch (padded_n(k.N)) {  // the fast Mamba-1 kernels it serves take state_dim <= 64
    case 8: { SSCAN_P1(8) break; }
    case 16: { SSCAN_P1(16) break; }
    case 32: { SSCAN_P1(32) break; }
    default: { SSCAN_P1(64) break; }
  }
#undef SSCAN_P1
}

template <typename T, bool SSD>
void dispatch_step(const TLK& k, int64_t batch, bool gate, hipStream_t s) {
  const dim3 blk(256);
#define SSCAN_STEP(NP)                                                                                   \
  {                                                                                                      \
    const dim3 grid((unsigned)((k.Dc * step_lanes<NP>() + 255) / 256), (unsigned)batch);                \
    if (gate) hipLaunchKernelGGL((tokenloop_step_kernel<T, NP, SSD, true>), grid, blk, 0, s, k);         \
    else hipLaunchKernelGGL((tokenloop_step_kernel<T, NP, SSD, false>), grid, blk, 0, s, k);             \
  }
  switch (padded_n(k.N)) {
    case 8: { SSCAN_STEP(8) break; }
    case 16: { SSCAN_STEP(16) break; }
    case 32: { SSCAN_STEP(32) break; }
    case 64: { SSCAN_STEP(64) break; }
    case 128: { SSCAN_STEP(128) break; }
    default: {  // Mamba-1 only, as in dispatch_scan
      if constexpr (!SSD) SSCAN_STEP(256)
      break;
    }
  }
#undef SSCAN_STEP
}

}  // namespace sscan
