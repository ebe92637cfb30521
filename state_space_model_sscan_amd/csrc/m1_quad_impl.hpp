// m1_quad_impl.hpp -- the Mamba-1 prompt scan with a quad of lanes per channel
// (instantiated in m1q_*.hip), for shapes with channels enough to give every SIMD
// two waves at four lanes per channel (the Falcon-Mamba-7b width and wider).
//
// Same recurrence as m1_row_impl.hpp ("Mamba", nnterp guide, opening paragraph and
// section "The values"; "Mamba", tokentrails lineage, "Code"; "Falcon-Mamba",
// "Where the norms sit" for the optional B/C norm):
//     dt  = softplus(dt_raw + dt_bias[c]);  A = -exp(A_log)
//     h_n = exp(dt * A[c, n]) * h_n + dt * B_n * x
//     y   = (sum_n C_n h_n + D[c] * x) * silu(z)      (gate optional)
//
// The scan is bound by VALU issue. A state update costs the same everywhere (a
// multiply for dt * A, the exp, a multiply for dt * x * B, the state FMA and the
// read-out FMA, where the exp issues at half rate); what a mapping adds on top is
// the per-token work of a channel and the sum of the read-out over the channel's
// lanes. With four lanes per channel (lane q holds state entries q N/4 .. q N/4 +
// N/4 - 1) the read-out sums over a quad: a transpose-reduce of two DPP stages per
// four tokens, against four stages per sixteen tokens with a 16-lane row, and each
// lane owns the per-token work (softplus, gate, store) of one token in four.
//  * A 256-thread block owns 64 channels of one batch row and walks the sequence in
//    64-token tiles. Each tile's x, dt_raw and z are loaded cooperatively in 16-byte
//    pieces of whole rows and staged raw in LDS; B and C are loaded a token quarter
//    per thread, normed when asked (a quad sum of squares), and staged as fp32.
//    The next tile's loads are in flight while a tile is computed; y leaves through
//    LDS in 16-byte pieces of whole rows.
//  * Lane q computes the step of token 4g + q of group g; at step s every lane of
//    the quad takes dt and dt * x of token 4g + s from lane s by a DPP quad
//    broadcast.
//  * Buffer resources are based at the tile's first token row and end at the
//    slice's last token, so rows past the end read zeros and drop their stores in
//    hardware; channel pieces past the width carry an out-of-range offset.
// The host uses it for state_dim 16, 32 or 64 with channels in whole 16-byte pieces.
#pragma once
#include <utility>

#include "m1_row_impl.hpp"

namespace sscan {

namespace quad {

// v of lane S of this lane's quad (DPP quad_perm [S, S, S, S]).
template <int S>
__device__ __forceinline__ float qb(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), S | (S << 2) | (S << 4) | (S << 6), 0xF,
                                                    0xF, false));
}

}  // namespace quad

template <typename T, int NP, bool GATE, bool STATES>
__global__ __launch_bounds__(256) void m1_quad_kernel(M1F k) {
  using namespace quad;
  constexpr int NPL = NP / 4;    // state entries per lane
  constexpr int TILE = 64;       // tokens per tile
  constexpr int CPB = 64;        // channels per block (16 per wave)
  constexpr uint32_t ES = sizeof(T);
  constexpr int EPP = 16 / ES;              // elements per 16-byte piece
  constexpr int PPR = CPB / EPP;            // pieces per tile row
  constexpr int PIT = TILE * PPR / 256;     // pieces per thread and tensor
  constexpr int RPI = 256 / PPR;            // tile rows per pass of the block
  // row pitch of the raw tiles (elements): bf16 rows 160 bytes apart put the four
  // token rows a wave reads at once on disjoint banks
  constexpr int XP = CPB + (ES == 2 ? 16 : 16);
  constexpr int NQ = NP / 4;                // B/C entries a staging thread takes (4 threads per token)
  constexpr int WQ = NQ * ES / 4;           // dwords of those entries
  __shared__ __attribute__((aligned(16))) T sA[3][TILE][XP];   // [x, dt_raw, z][token][channel]
  __shared__ __attribute__((aligned(16))) T sY[TILE][XP];
  __shared__ __attribute__((aligned(16))) float sBC[2][TILE][NP];  // [B, C][token][entry]

  const int tid = threadIdx.x;
  const int l = tid & 63, w = tid >> 6;
  const int q = l & 3;                   // lane in the quad
  const int cl = 16 * w + (l >> 2);      // channel in the block
  const int64_t ncb = (k.Dc + CPB - 1) / CPB;
  const int64_t lb = xcd_local_order(blockIdx.x, (int64_t)gridDim.x);
  const int64_t cb = lb % ncb;
  const int s = (int)((lb / ncb) % k.nslices);
  const int64_t b = lb / (ncb * k.nslices);
  const int64_t c0 = cb * CPB;
  const int64_t c = c0 + cl;
  const bool active = c < k.Dc;
  const int64_t cc = active ? c : k.Dc - 1;
  // token indices fit in 32 bits: the host guarantees L*Dc*ES < 2^31
  const int t_begin = s * k.slice_len;
  const int t_end = (int)min(k.L, (int64_t)t_begin + k.slice_len);
  const int g = (int)(c0 / k.per_group);  // the host guarantees one group per block
  const int n0 = q * NPL;

  // cooperative tile I/O: piece p of row r (+ RPI it) for x, dt_raw, z and y
  const int pr = tid / PPR, pp = tid % PPR;
  const uint32_t row_bytes = (uint32_t)(k.Dc * ES);
  const uint32_t bc_row = (uint32_t)(k.G * k.N * ES);
  const char* xb = (const char*)k.x + b * k.L * k.Dc * ES;
  const char* db = (const char*)k.dt + b * k.L * k.Dc * ES;
  const char* zb = GATE ? (const char*)k.z + b * k.L * k.Dc * ES : xb;
  char* yb = (char*)k.y + b * k.L * k.Dc * ES;
  const char* Bb = (const char*)k.B + b * k.L * k.G * k.N * ES;
  const char* Cb = (const char*)k.C + b * k.L * k.G * k.N * ES;
  auto tile_rsrc = [&](const char* base, int t0, uint32_t row) {
    const int left = t_end - t0;
    return make_rsrc(base + (int64_t)t0 * row, left > 0 ? (uint32_t)left * row : 0u);
  };
  // channels c0 + EPP pp .. of row pr: all inside the width or all past it
  const uint32_t vx = c0 + EPP * pp < k.Dc ? (uint32_t)(pr * row_bytes + (c0 + EPP * pp) * ES) : kOOB;
  // B/C: token tb_ = tid / 4, entries tq_ NQ .. of group g
  const int tb_ = tid >> 2, tq_ = tid & 3;
  const uint32_t vb = (uint32_t)(tb_ * bc_row + (g * k.N + tq_ * NQ) * ES);

  float A2[NPL], h[NPL];
#pragma unroll
  for (int i = 0; i < NPL; ++i) {
    A2[i] = -expf(k.A_log[cc * k.N + n0 + i]) * kLog2e;
    h[i] = k.h0 ? k.h0[(b * k.Dc + cc) * k.N + n0 + i] : 0.0f;
  }
  for (int j = 0; j < s; ++j) {  // carry in from the slices before this one
    const int64_t base = (b * k.nslices + j) * k.Dc + cc;
    const float sdt = k.ws_sdt[base];
#pragma unroll
    for (int i = 0; i < NPL; ++i) h[i] = fmaf(fast_exp2(A2[i] * sdt), h[i], k.ws_h[base * k.N + n0 + i]);
  }
  const float bias = k.dt_bias[cc];
  const float Dv = k.D[cc];
  const float inv_n = 1.0f / (float)k.N;
  const bool bc_norm = k.bc_eps > 0.0f;

  struct Raw {
    u32x4 a[GATE ? 3 : 2][PIT];
    RawVec<WQ> bq, cq;
  };
  auto load_raw = [&](Raw& r, int t0) {
    const __amdgpu_buffer_rsrc_t rx = tile_rsrc(xb, t0, row_bytes), rd = tile_rsrc(db, t0, row_bytes);
#pragma unroll
    for (int it = 0; it < PIT; ++it) {
      const uint32_t o = vx == kOOB ? kOOB : vx + it * RPI * row_bytes;
      r.a[0][it] = __builtin_amdgcn_raw_buffer_load_b128(rx, (int)o, 0, 0);
      r.a[1][it] = __builtin_amdgcn_raw_buffer_load_b128(rd, (int)o, 0, 0);
    }
    if constexpr (GATE) {
      const __amdgpu_buffer_rsrc_t rz = tile_rsrc(zb, t0, row_bytes);
#pragma unroll
      for (int it = 0; it < PIT; ++it)
        r.a[2][it] = __builtin_amdgcn_raw_buffer_load_b128(rz, (int)(vx == kOOB ? kOOB : vx + it * RPI * row_bytes), 0,
                                                           0);
    }
    r.bq.load(tile_rsrc(Bb, t0, bc_row), vb);
    r.cq.load(tile_rsrc(Cb, t0, bc_row), vb);
  };
  auto stage = [&](Raw& r) {
#pragma unroll
    for (int a = 0; a < (GATE ? 3 : 2); ++a)
#pragma unroll
      for (int it = 0; it < PIT; ++it) *(u32x4*)&sA[a][pr + it * RPI][EPP * pp] = r.a[a][it];
    float bv[NQ], cv[NQ];
    r.bq.template unpack<T>(bv);
    r.cq.template unpack<T>(cv);
    float sb = 0.0f, sc = 0.0f;
    if (bc_norm) {
#pragma unroll
      for (int j = 0; j < NQ; ++j) {
        sb = fmaf(bv[j], bv[j], sb);
        sc = fmaf(cv[j], cv[j], sc);
      }
      sb += dpp_f<0xB1>(sb);  // sum over the token's four threads
      sc += dpp_f<0xB1>(sc);
      sb += dpp_f<0x4E>(sb);
      sc += dpp_f<0x4E>(sc);
      const float ib = __builtin_amdgcn_rsqf(fmaf(sb, inv_n, k.bc_eps));
      const float ic = __builtin_amdgcn_rsqf(fmaf(sc, inv_n, k.bc_eps));
#pragma unroll
      for (int j = 0; j < NQ; ++j) {
        bv[j] *= ib;
        cv[j] *= ic;
      }
    }
#pragma unroll
    for (int j = 0; j < NQ; j += 4) {
      *(f32x4*)&sBC[0][tb_][tq_ * NQ + j] = f32x4{bv[j], bv[j + 1], bv[j + 2], bv[j + 3]};
      *(f32x4*)&sBC[1][tb_][tq_ * NQ + j] = f32x4{cv[j], cv[j + 1], cv[j + 2], cv[j + 3]};
    }
  };
  auto store_y = [&](int t0) {
    const __amdgpu_buffer_rsrc_t ry = tile_rsrc(yb, t0, row_bytes);
#pragma unroll
    for (int it = 0; it < PIT; ++it)
      __builtin_amdgcn_raw_buffer_store_b128(*(const u32x4*)&sY[pr + it * RPI][EPP * pp], ry,
                                             (int)(vx == kOOB ? kOOB : vx + it * RPI * row_bytes), 0, 0);
  };

  // Group j (tokens t0 + 4j .. t0 + 4j + 3) of the tile in LDS. TAIL: the tile
  // may run past the slice's end (only the last tile does), so its steps are masked.
  auto compute_group = [&](int t0, int j, auto tail) {
    constexpr bool TAIL = decltype(tail)::value;
    const int tl = 4 * j + q;  // this lane's token in the tile
    const float xv = to_f<T>(sA[0][tl][cl]);
    const float sp = softplus_fast(to_f<T>(sA[1][tl][cl]) + bias);
    const float dtv = (!TAIL || t0 + tl < t_end) ? sp : 0.0f;  // a token past the end is a zero step
    const float dtx = dtv * xv;
    float p[4];
    static_for<4>([&](auto S) {
      constexpr int st = decltype(S)::value;
      const float dk = qb<st>(dtv);
      const float xk = qb<st>(dtx);
      float bv[NPL], cv[NPL];
#pragma unroll
      for (int i = 0; i < NPL; i += 4) {
        const f32x4 b4 = *(const f32x4*)&sBC[0][4 * j + st][n0 + i];
        const f32x4 c4 = *(const f32x4*)&sBC[1][4 * j + st][n0 + i];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          bv[i + e] = b4[e];
          cv[i + e] = c4[e];
        }
      }
      float acc = 0.0f;
#pragma unroll
      for (int i = 0; i < NPL; ++i) {
        h[i] = fmaf(fast_exp2(dk * A2[i]), h[i], xk * bv[i]);
        acc = i == 0 ? cv[i] * h[i] : fmaf(cv[i], h[i], acc);
      }
      p[st] = acc;
      if constexpr (STATES) {
        const int tk = t0 + 4 * j + st;
        if (tk < t_end && active) {
          float* sp_ = k.states + ((b * k.L + tk) * k.Dc + c) * k.N + n0;
#pragma unroll
          for (int i = 0; i < NPL; i += 4) *(f32x4*)(sp_ + i) = f32x4{h[i], h[i + 1], h[i + 2], h[i + 3]};
        }
      }
    });
    float yv = kreduce<4>(p, q) + Dv * xv;
    if (GATE) yv *= silu(to_f<T>(sA[2][tl][cl]));
    sY[tl][cl] = from_f<T>(yv);
  };

  // Per tile: barrier (the previous tile's compute is done: LDS free, its y
  // complete); stage this tile (its loads were issued a tile ago); store the
  // previous tile's y; issue the next tile's loads; barrier; compute.
  Raw raw;
  load_raw(raw, t_begin);
  for (int t0 = t_begin; t0 < t_end; t0 += TILE) {
    __syncthreads();
    stage(raw);
    if (t0 > t_begin) store_y(t0 - TILE);
    load_raw(raw, t0 + TILE);
    __syncthreads();
    if (t0 + TILE <= t_end) {  // uniform: every token of the tile is in the slice
#pragma unroll 4
      for (int j = 0; j < TILE / 4; ++j) compute_group(t0, j, std::false_type{});
    } else {
      for (int j = 0; j < TILE / 4; ++j) compute_group(t0, j, std::true_type{});
    }
  }
  __syncthreads();
  if (t_end > t_begin) store_y(t_begin + ((t_end - t_begin - 1) / TILE) * TILE);

  if (s == k.nslices - 1 && active) {
#pragma unroll
    for (int i = 0; i < NPL; i += 4)
      *(f32x4*)(k.h_out + (b * k.Dc + c) * k.N + n0 + i) = f32x4{h[i], h[i + 1], h[i + 2], h[i + 3]};
  }
}

template <typename T, int NP>
void launch_m1_quad_np(const M1F& k, bool gate, bool states, dim3 grid, hipStream_t s) {
  const dim3 blk(256);
  if (gate && states) hipLaunchKernelGGL((m1_quad_kernel<T, NP, true, true>), grid, blk, 0, s, k);
  else if (gate) hipLaunchKernelGGL((m1_quad_kernel<T, NP, true, false>), grid, blk, 0, s, k);
  else if (states) hipLaunchKernelGGL((m1_quad_kernel<T, NP, false, true>), grid, blk, 0, s, k);
  else hipLaunchKernelGGL((m1_quad_kernel<T, NP, false, false>), grid, blk, 0, s, k);
}

}  // namespace sscan
