// m1_fast_impl.hpp -- the Mamba-1 prompt scan kernel for gfx950 (instantiated in m1_fast_*.hip).
//
// Computes, per channel c and state entry n ("Mamba", nnterp guide, opening
// paragraph and section "The values"; "Mamba", tokentrails lineage, "Code";
// "Falcon-Mamba", "Where the norms sit" for the optional B/C norm):
//     dt  = softplus(dt_raw + dt_bias[c]);  A = -exp(A_log)
//     h_n = exp(dt * A[c, n]) * h_n + dt * B_n * x
//     y   = (sum_n C_n h_n + D[c] * x) * silu(z)      (gate optional)
//
// On MI355X this scan is bound by VALU issue, not by HBM: every state update
// needs dt*A, exp2, dt*x*B, the state FMA and the read-out FMA, and v_exp_f32
// runs at half rate. The kernel spends the VALU on that and little else:
//  * K lanes share a channel (K = 1, 2 or 4), each holding state_dim/K entries
//    in registers, so that a grid of batch*channels*K lanes covers every SIMD.
//    The per-token work of a channel (loads, softplus, gate, store) is spread
//    over its K lanes: lane q handles tokens t0+q, t0+q+K, ...; dt and dt*x of
//    each token reach the other lanes by DPP quad broadcast, and the partial
//    read-outs are summed back to the owning lane by a DPP transpose-reduce.
//  * x, dt_raw, z and y go through raw buffer instructions: the batch row is
//    the resource, the lane's channel a fixed byte offset, and the token row a
//    uniform scalar offset, so no per-token address arithmetic reaches the
//    VALU. Lanes past the last channel carry an out-of-range offset, which the
//    hardware turns into loads of zero and dropped stores.
//  * x, dt_raw and z of a lane's next 8 tokens (a block of 8*K tokens) are in
//    flight while the current block is computed. Every load is issued
//    unconditionally (a token past the end reads zeros through an out-of-range
//    offset) so that control flow stays uniform and the compiler's wait counts
//    let each prefetch run across a whole block.
//  * B and C of a tile of tokens (shared by every channel of the group) are
//    normed, converted to fp32 and staged in LDS once; the raw values of the
//    next tile are loaded during the current one.
//  * exp(dt*A) is evaluated as exp2(dt * (A*log2 e)) with A*log2 e per lane.
// Long sequences with few channels are cut into slices: the token-loop pass 1
// scans each slice from zero and stores its end state and step sum, and this
// kernel starts slice s from the combined carry.
#pragma once
#include "device_common.hpp"
#include "launch.hpp"

namespace sscan {

struct M1F {
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
  const float* ws_h;    // [batch, nslices, Dc, N] slice end states (nslices > 1)
  const float* ws_sdt;  // [batch, nslices, Dc]   slice step sums
  int64_t L, Dc, per_group;
  int N, G, nslices, slice_len;
  float bc_eps;
};

constexpr uint32_t kOOB = 0x80000000u;  // a buffer offset past any resource this kernel builds

// DPP quad permutation: lane i of each group of 4 takes lane sel[i] (2 bits per lane).
#define SSCAN_QPERM(v, sel) __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), (sel), 0xF, 0xF, false))

// Value of lane `src` of this lane's K-group (K = 1, 2, 4; groups aligned to quads).
template <int K>
__device__ __forceinline__ float kbcast(float v, int src) {
  if constexpr (K == 1) {
    return v;
  } else if constexpr (K == 2) {
    return src == 0 ? SSCAN_QPERM(v, 0xA0) : SSCAN_QPERM(v, 0xF5);  // [0,0,2,2] / [1,1,3,3]
  } else {
    switch (src) {
      case 0: return SSCAN_QPERM(v, 0x00);
      case 1: return SSCAN_QPERM(v, 0x55);
      case 2: return SSCAN_QPERM(v, 0xAA);
      default: return SSCAN_QPERM(v, 0xFF);
    }
  }
}

// yp[k] holds this lane's partial read-out for token k of the group; returns the
// total over the K lanes for token q (this lane's own token).
template <int K>
__device__ __forceinline__ float kreduce(const float (&yp)[K], int q) {
  if constexpr (K == 1) {
    return yp[0];
  } else if constexpr (K == 2) {
    const float keep = q ? yp[1] : yp[0];
    const float send = q ? yp[0] : yp[1];
    return keep + SSCAN_QPERM(send, 0xB1);  // swap within pairs [1,0,3,2]
  } else {
    const bool o = q & 1;
    const float k0 = o ? yp[1] : yp[0], s0 = o ? yp[0] : yp[1];
    const float k1 = o ? yp[3] : yp[2], s1 = o ? yp[2] : yp[3];
    const float r0 = k0 + SSCAN_QPERM(s0, 0xB1);  // tokens with bit0 == q&1, summed over q, q^1
    const float r1 = k1 + SSCAN_QPERM(s1, 0xB1);
    const bool t = q & 2;
    const float kb = t ? r1 : r0, sb = t ? r0 : r1;
    return kb + SSCAN_QPERM(sb, 0x4E);  // [2,3,0,1]
  }
}

// Raw buffer access to one activation element (bf16 or f32).
template <typename T> struct BufAct;
template <> struct BufAct<uint16_t> {
  // A loaded element in the low half of a register whose high half is left
  // undefined (the conversion shifts it out), so no zero-extension is needed
  // between the load and the conversion.
  using Raw = uint32_t;
  typedef short s16x2 __attribute__((ext_vector_type(2)));
  static __device__ __forceinline__ Raw ldr(__amdgpu_buffer_rsrc_t r, uint32_t voff) {
    s16x2 v;
    v[0] = (short)__builtin_amdgcn_raw_buffer_load_b16(r, (int)voff, 0, 0);
    return __builtin_bit_cast(uint32_t, v);
  }
  static __device__ __forceinline__ float fr(Raw raw) { return __uint_as_float(raw << 16); }
  static __device__ __forceinline__ uint32_t ld(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    return __builtin_amdgcn_raw_buffer_load_b16(r, (int)voff, (int)soff, 0);
  }
  static __device__ __forceinline__ float f(uint32_t raw) { return __uint_as_float(raw << 16); }
  static __device__ __forceinline__ void st(float v, __amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    __builtin_amdgcn_raw_buffer_store_b16(f32_to_bf16(v), r, (int)voff, (int)soff, 0);
  }
};
template <> struct BufAct<float> {
  using Raw = uint32_t;
  static __device__ __forceinline__ Raw ldr(__amdgpu_buffer_rsrc_t r, uint32_t voff) {
    return __builtin_amdgcn_raw_buffer_load_b32(r, (int)voff, 0, 0);
  }
  static __device__ __forceinline__ float fr(Raw raw) { return __uint_as_float(raw); }
  static __device__ __forceinline__ uint32_t ld(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    return __builtin_amdgcn_raw_buffer_load_b32(r, (int)voff, (int)soff, 0);
  }
  static __device__ __forceinline__ float f(uint32_t raw) { return __uint_as_float(raw); }
  static __device__ __forceinline__ void st(float v, __amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, (int)voff, (int)soff, 0);
  }
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

template <int NP> constexpr int m1_tile() { return 64; }

// Raw B and C of one token (lane = token of a tile): NP values each, as loaded.
template <typename T, int NP>
struct RawBC {
  uint32_t b[NP], c[NP];
};

// Loads B and C of token `tok` (batch-row relative) for group g through buffer
// resources over the batch row; a token past t_end reads zeros (out-of-range
// offset), and so do state entries past N.
template <typename T, int NP>
__device__ __forceinline__ void load_bc(const M1F& k, __amdgpu_buffer_rsrc_t rb, __amdgpu_buffer_rsrc_t rc, int64_t tok,
                                        int64_t t_end, int g, RawBC<T, NP>& r) {
  constexpr uint32_t ES = sizeof(T);
  const uint32_t vo = tok < t_end ? (uint32_t)((tok * k.G + g) * k.N * ES) : kOOB;
  if (k.N == NP && (NP * ES) % 16 == 0) {
    // whole rows of 16-byte pieces
#pragma unroll
    for (int p = 0; p < (int)(NP * ES / 16); ++p) {
      const auto vb = __builtin_amdgcn_raw_buffer_load_b128(rb, (int)vo, p * 16, 0);
      const auto vc = __builtin_amdgcn_raw_buffer_load_b128(rc, (int)vo, p * 16, 0);
      constexpr int per = 16 / ES;  // elements per piece
#pragma unroll
      for (int e = 0; e < per; ++e) {
        const uint32_t wb = vb[(e * ES) / 4], wc = vc[(e * ES) / 4];
        r.b[p * per + e] = ES == 4 ? wb : ((e & 1) ? (wb >> 16) : (wb & 0xffffu));
        r.c[p * per + e] = ES == 4 ? wc : ((e & 1) ? (wc >> 16) : (wc & 0xffffu));
      }
    }
  } else {
#pragma unroll
    for (int n = 0; n < NP; ++n) {
      const bool in = n < k.N;
      const uint32_t vn = in ? vo + (uint32_t)(n * ES) : kOOB;
      r.b[n] = BufAct<T>::ld(rb, vn, 0);
      r.c[n] = BufAct<T>::ld(rc, vn, 0);
    }
  }
}

template <typename T, int NP>
__device__ __forceinline__ void store_bc(const M1F& k, const RawBC<T, NP>& r, float (*sBC)[2][NP], int slot) {
  float bv[NP], cv[NP];
  float sb = 0.0f, sc = 0.0f;
#pragma unroll
  for (int n = 0; n < NP; ++n) {
    bv[n] = BufAct<T>::f(r.b[n]);
    cv[n] = BufAct<T>::f(r.c[n]);
    sb = fmaf(bv[n], bv[n], sb);
    sc = fmaf(cv[n], cv[n], sc);
  }
  if (k.bc_eps > 0.0f) {
    const float ib = 1.0f / sqrtf(sb / (float)k.N + k.bc_eps);
    const float ic = 1.0f / sqrtf(sc / (float)k.N + k.bc_eps);
#pragma unroll
    for (int n = 0; n < NP; ++n) {
      bv[n] *= ib;
      cv[n] *= ic;
    }
  }
#pragma unroll
  for (int n = 0; n < NP; ++n) {
    sBC[slot][0][n] = bv[n];
    sBC[slot][1][n] = cv[n];
  }
}

template <int GPB>
struct RawTok {
  uint32_t x[GPB], d[GPB], z[GPB];
};

template <typename T, int NP, int K, bool GATE, bool STATES>
__global__ __launch_bounds__(64) void m1_fast_kernel(M1F k) {
  constexpr int NPL = NP / K;  // state entries per lane
  constexpr int CPW = 64 / K;  // channels per wave
  constexpr int GPB = 8;       // token groups per register block: 8 own tokens per lane
  constexpr int BT = GPB * K;  // tokens per register block
  constexpr int TILE = m1_tile<NP>();
  constexpr int NB = TILE / BT;  // register blocks per tile
  constexpr uint32_t ES = sizeof(T);
  constexpr bool PREF = NP <= 16;  // raw B/C of the next tile held in registers during a tile
  static_assert(TILE % (2 * BT) == 0, "a tile holds an even number of blocks");
  __shared__ float sBC[TILE][2][NP];

  const int lane = threadIdx.x;
  const int q = lane % K;
  // 1-D grid of (channel block, slice, batch); neighbouring channel blocks share
  // 128-byte lines of x/dt/z/y, so they go to one XCD
  const int64_t ncb = (k.Dc + CPW - 1) / CPW;
  const int64_t lb = xcd_local_order(blockIdx.x, (int64_t)gridDim.x);
  const int64_t cb = lb % ncb;
  const int s = (int)((lb / ncb) % k.nslices);
  const int64_t b = lb / (ncb * k.nslices);
  const int64_t c0 = cb * CPW;
  const int64_t c = c0 + lane / K;
  const bool active = c < k.Dc;
  const int64_t cc = active ? c : k.Dc - 1;
  const int64_t t_begin = (int64_t)s * k.slice_len;
  const int64_t t_end = min(k.L, t_begin + (int64_t)k.slice_len);
  const int g = (int)(c0 / k.per_group);  // the host guarantees one group per wave
  const int n0 = q * NPL;

  // Buffer resources over this batch row; the host guarantees L*Dc*ES < 2^31.
  const uint32_t row_bytes = (uint32_t)(k.Dc * ES);
  const uint32_t batch_bytes = (uint32_t)(k.L * k.Dc * ES);
  const int64_t boff = b * k.L * k.Dc;
  const __amdgpu_buffer_rsrc_t rx = make_rsrc((const T*)k.x + boff, batch_bytes);
  const __amdgpu_buffer_rsrc_t rd = make_rsrc((const T*)k.dt + boff, batch_bytes);
  const __amdgpu_buffer_rsrc_t rz = make_rsrc(GATE ? (const T*)k.z + boff : (const T*)k.x, batch_bytes);
  const __amdgpu_buffer_rsrc_t ry = make_rsrc((T*)k.y + boff, batch_bytes);
  const uint32_t bc_bytes = (uint32_t)(k.L * k.G * k.N * ES);
  const int64_t bcoff = b * k.L * k.G * k.N;
  const __amdgpu_buffer_rsrc_t rB = make_rsrc((const T*)k.B + bcoff, bc_bytes);
  const __amdgpu_buffer_rsrc_t rC = make_rsrc((const T*)k.C + bcoff, bc_bytes);
  // the lane's own element: token row q of a group, channel c
  const uint32_t lane_off = active ? (uint32_t)((q * k.Dc + c) * ES) : kOOB;

  float A2[NPL], h[NPL];
#pragma unroll
  for (int i = 0; i < NPL; ++i) {
    const int n = n0 + i;
    A2[i] = n < k.N ? -expf(k.A_log[cc * k.N + n]) * kLog2e : 0.0f;
    h[i] = (k.h0 && n < k.N) ? k.h0[(b * k.Dc + cc) * k.N + n] : 0.0f;
  }
  for (int j = 0; j < s; ++j) {  // carry in from the slices before this one
    const int64_t base = (b * k.nslices + j) * k.Dc + cc;
    const float sdt = k.ws_sdt[base];
#pragma unroll
    for (int i = 0; i < NPL; ++i)
      if (n0 + i < k.N) h[i] = fmaf(fast_exp2(A2[i] * sdt), h[i], k.ws_h[base * k.N + n0 + i]);
  }
  const float bias = k.dt_bias[cc];
  const float Dv = k.D[cc];

  // Loads of the block starting at token tb: group gi, lane q reads token tb + gi*K + q.
  // Unconditional: tokens at or past t_end read zeros through an out-of-range offset.
  auto load_block = [&](RawTok<GPB>& r, int64_t tb) {
#pragma unroll
    for (int gi = 0; gi < GPB; ++gi) {
      const int64_t tq = tb + gi * K + q;
      const uint32_t soff = tb + gi * K < t_end ? (uint32_t)((tb + gi * K) * row_bytes) : 0u;
      const uint32_t vo = tq < t_end ? lane_off : kOOB;
      r.x[gi] = BufAct<T>::ld(rx, vo, soff);
      r.d[gi] = BufAct<T>::ld(rd, vo, soff);
      if (GATE) r.z[gi] = BufAct<T>::ld(rz, vo, soff);
    }
  };

  // One block of BT tokens from tile slot tt0 on.
  auto compute_block = [&](const RawTok<GPB>& cur, int64_t tb, int tt0) {
#pragma unroll
    for (int gi = 0; gi < GPB; ++gi) {
      const int64_t tq = tb + gi * K + q;  // this lane's token in group gi
      const bool vq = tq < t_end;
      const float xv = BufAct<T>::f(cur.x[gi]);
      const float sp = softplus_fast(BufAct<T>::f(cur.d[gi]) + bias);
      const float dtv = vq ? sp : 0.0f;  // a token past the end is a zero step
      const float dtx = dtv * xv;
      float yp_[K];
#pragma unroll
      for (int kk = 0; kk < K; ++kk) {
        const float dk = kbcast<K>(dtv, kk);
        const float xk = kbcast<K>(dtx, kk);
        const int slot = tt0 + gi * K + kk;
        const float* Bs = &sBC[slot][0][n0];
        const float* Cs = &sBC[slot][1][n0];
        float acc = 0.0f;
#pragma unroll
        for (int i = 0; i < NPL; ++i) {
          h[i] = fmaf(fast_exp2(dk * A2[i]), h[i], xk * Bs[i]);
          acc = fmaf(Cs[i], h[i], acc);
        }
        yp_[kk] = acc;
        if (STATES) {
          const int64_t tk = tb + gi * K + kk;
          if (tk < t_end && active) {
            float* sp_ = k.states + ((b * k.L + tk) * k.Dc + c) * k.N + n0;
#pragma unroll
            for (int i = 0; i < NPL; ++i)
              if (n0 + i < k.N) sp_[i] = h[i];
          }
        }
      }
      float yv = kreduce<K>(yp_, q) + Dv * xv;
      if (GATE) yv *= silu(BufAct<T>::f(cur.z[gi]));
      const uint32_t soff = tb + gi * K < t_end ? (uint32_t)((tb + gi * K) * row_bytes) : 0u;
      BufAct<T>::st(yv, ry, vq ? lane_off : kOOB, soff);
    }
  };

  RawBC<T, NP> rbc;
  if (PREF && lane < TILE) load_bc<T, NP>(k, rB, rC, t_begin + lane, t_end, g, rbc);
  RawTok<GPB> ra, rb;
  load_block(ra, t_begin);
  for (int64_t t0 = t_begin; t0 < t_end; t0 += TILE) {
    // this tile's B/C into LDS; with PREF they are already in registers and the
    // next tile's are loaded while this one is computed
    __syncthreads();
    if (!PREF && lane < TILE) load_bc<T, NP>(k, rB, rC, t0 + lane, t_end, g, rbc);
    if (lane < TILE) store_bc<T, NP>(k, rbc, sBC, lane);
    __syncthreads();
    if (PREF && lane < TILE) load_bc<T, NP>(k, rB, rC, t0 + TILE + lane, t_end, g, rbc);
#pragma unroll
    for (int jb = 0; jb < NB; jb += 2) {
      const int64_t tb = t0 + jb * BT;
      load_block(rb, tb + BT);
      compute_block(ra, tb, jb * BT);
      load_block(ra, tb + 2 * BT);
      compute_block(rb, tb + BT, (jb + 1) * BT);
    }
  }

  if (s == k.nslices - 1 && active) {
#pragma unroll
    for (int i = 0; i < NPL; ++i)
      if (n0 + i < k.N) k.h_out[(b * k.Dc + c) * k.N + n0 + i] = h[i];
  }
}

template <typename T, int NP>
void launch_m1_np(const M1F& k, int K, bool gate, bool states, dim3 grid, hipStream_t s) {
  const dim3 blk(64);
#define SSCAN_M1(KK)                                                                             \
  if (gate && states) hipLaunchKernelGGL((m1_fast_kernel<T, NP, KK, true, true>), grid, blk, 0, s, k);    \
  else if (gate) hipLaunchKernelGGL((m1_fast_kernel<T, NP, KK, true, false>), grid, blk, 0, s, k);        \
  else if (states) hipLaunchKernelGGL((m1_fast_kernel<T, NP, KK, false, true>), grid, blk, 0, s, k);      \
  else hipLaunchKernelGGL((m1_fast_kernel<T, NP, KK, false, false>), grid, blk, 0, s, k);
  if constexpr (NP < 64) {
    if (K == 1) { SSCAN_M1(1) return; }
  }
  if (K == 2) { SSCAN_M1(2) }
  else { SSCAN_M1(4) }
#undef SSCAN_M1
}

}  // namespace sscan
