// m1_row_impl.hpp -- the Mamba-1 prompt scan with one 16-lane DPP row per channel
// (instantiated in m1r_*.hip).
//
// Same recurrence as m1_fast_impl.hpp ("Mamba", nnterp guide, opening paragraph
// and section "The values"; "Mamba", tokentrails lineage, "Code"; "Falcon-Mamba",
// "Where the norms sit" for the optional B/C norm):
//     dt  = softplus(dt_raw + dt_bias[c]);  A = -exp(A_log)
//     h_n = exp(dt * A[c, n]) * h_n + dt * B_n * x
//     y   = (sum_n C_n h_n + D[c] * x) * silu(z)      (gate optional)
//
// The scan is VALU-bound on MI355X, and at the Mamba-130m width four lanes per
// channel give fewer waves than the chip has SIMDs. This kernel gives every
// channel a whole 16-lane row of a wave, lane n holding state entries n, n+16, ..,
// which quadruples the waves (three per SIMD for a batch of 8 at width 1536).
// A 256-thread block owns 16 channels and walks the sequence in 128-token tiles:
//  * Each tile's x, dt_raw, z, B and C are loaded cooperatively, a thread reading
//    4 neighbouring channels (or state entries) of one token in a single 8- or
//    16-byte load, converted to fp32 and written to LDS: x/dt/z as [token][channel],
//    B/C transposed as [state][token]. The next tile's loads are in flight while a
//    tile is computed. (Loading the scan layout straight from memory would make
//    every instruction touch 16 token rows; measured, that is twice as slow.)
//  * Lane n of a channel's row takes token n of a 16-token group from LDS and
//    computes its softplus and dt*x once. At step s every lane takes dt and dt*x
//    of token s from lane s of its row by DPP row_newbcast, which the compiler
//    folds into the multiplies that consume them.
//  * Each lane keeps its partial read-out C_n h_n for the 16 tokens of a group; a
//    transpose-reduce over the row (four DPP exchange stages: lane n with n^8 and
//    n^4 as bank-masked DPP adds, then n^2 and n^1 with selects) leaves the full
//    sum for token n in lane n, which adds D*x, applies the gate and writes y to
//    LDS; the block stores the tile's y as 8/16-byte pieces.
//  * Every buffer resource is based at the tile's first token row and ends at
//    the slice's last token, so rows past the end read zeros and drop their
//    stores in hardware, and per-lane offsets stay fixed over the whole scan.
// The host uses this kernel when state_dim is 16, 32 or 64 and channels are a
// multiple of 4 (so a thread's 4 channels are all inside the row or all past it).
#pragma once
#include <type_traits>
#include <utility>

#include "m1_fast_impl.hpp"

namespace sscan {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// v of lane S of this lane's row (DPP row_newbcast).
template <int S>
__device__ __forceinline__ float row_bcast(float v) {
  return dpp_f<0x150 + S>(v);
}

template <typename F, int... S>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, S...>) {
  (f(std::integral_constant<int, S>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// Contiguous raw loads of W dwords (1, 2 or a multiple of 4) through a buffer resource.
template <int W>
struct RawVec {
  uint32_t w[W];
  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t r, uint32_t voff) {
    if constexpr (W == 1) {
      w[0] = __builtin_amdgcn_raw_buffer_load_b32(r, (int)voff, 0, 0);
    } else if constexpr (W == 2) {
      const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(r, (int)voff, 0, 0);
      w[0] = v[0];
      w[1] = v[1];
    } else {
      static_assert(W % 4 == 0, "wide pieces are whole 16-byte loads");
#pragma unroll
      for (int p = 0; p < W / 4; ++p) {
        const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)(voff + 16 * p), 0, 0);
        w[4 * p + 0] = v[0];
        w[4 * p + 1] = v[1];
        w[4 * p + 2] = v[2];
        w[4 * p + 3] = v[3];
      }
    }
  }
  // The elements as fp32 (2 per dword for bf16, 1 for fp32); the asm keeps the
  // use here rather than letting the compiler hoist it to just after the load.
  template <typename T>
  __device__ __forceinline__ void unpack(float* out) {
#pragma unroll
    for (int i = 0; i < W; ++i) asm volatile("" : "+v"(w[i]));
    if constexpr (sizeof(T) == 2) {
#pragma unroll
      for (int i = 0; i < W; ++i) {
        out[2 * i] = __uint_as_float(w[i] << 16);
        out[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
      }
    } else {
#pragma unroll
      for (int i = 0; i < W; ++i) out[i] = __uint_as_float(w[i]);
    }
  }
};

namespace quad {
// activations as stored (bf16 bits or fp32) to fp32 and back (round to nearest even)
template <typename T> __device__ __forceinline__ float to_f(T v);
template <> __device__ __forceinline__ float to_f<uint16_t>(uint16_t v) { return bf16_to_f32(v); }
template <> __device__ __forceinline__ float to_f<float>(float v) { return v; }
template <typename T> __device__ __forceinline__ T from_f(float v);
template <> __device__ __forceinline__ uint16_t from_f<uint16_t>(float v) { return f32_to_bf16(v); }
template <> __device__ __forceinline__ float from_f<float>(float v) { return v; }
}  // namespace quad

template <typename T, int NP, bool GATE, bool STATES>
__global__ __launch_bounds__(256) void m1_row_kernel(M1F k) {
  constexpr int NPL = NP / 16;  // state entries per lane
  constexpr int NQ = NP / 4;    // B/C entries a thread stages (4 threads per token)
  constexpr int RT = 2;         // token rows a thread stages per tile
  constexpr int TILE = 64 * RT;
  constexpr int TP = TILE + 4;  // LDS pitch (floats) of a state entry's row of tokens
  // LDS pitch (elements) of a token's 16 channels, kept as loaded: 40 bytes for
  // bf16, so that the 16 token rows a wave reads at once fall on distinct banks
  constexpr int XP = 20;
  constexpr uint32_t ES = sizeof(T);
  constexpr int WA = ES;           // dwords of 4 activations
  constexpr int WQ = NQ * ES / 4;  // dwords of a thread's B (or C) entries
  __shared__ __attribute__((aligned(16))) float sBC[2][NP][TP];  // [B, C][entry][token]
  __shared__ __attribute__((aligned(16))) T sX[3][TILE][XP];      // [x, dt, z][token][channel]
  __shared__ __attribute__((aligned(16))) T sY[TILE][XP];         // [token][channel]

  const int tid = threadIdx.x;
  const int n = tid & 15;   // lane in the channel's row; token of a group
  const int cl = tid >> 4;  // channel within the block
  const int64_t ncb = (k.Dc + 15) / 16;
  const int64_t lb = xcd_local_order(blockIdx.x, (int64_t)gridDim.x);
  const int64_t cb = lb % ncb;
  const int s = (int)((lb / ncb) % k.nslices);
  const int64_t b = lb / (ncb * k.nslices);
  const int64_t c0 = cb * 16;
  const int64_t c = c0 + cl;
  const bool active = c < k.Dc;
  const int64_t cc = active ? c : k.Dc - 1;
  // token indices fit in 32 bits: the host guarantees L*Dc*ES < 2^31
  const int t_begin = s * k.slice_len;
  const int t_end = (int)min(k.L, (int64_t)t_begin + k.slice_len);
  const int g = (int)(c0 / k.per_group);  // the host guarantees one group per block

  // Cooperative tile I/O: thread -> token row tr of the tile, quarter tq.
  const int tr = tid >> 2, tq = tid & 3;
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
  // channels c0+4tq .. c0+4tq+3 of token row tr (all in the row or all past it)
  const uint32_t vx = c0 + 4 * tq < k.Dc ? (uint32_t)(tr * row_bytes + (c0 + 4 * tq) * ES) : kOOB;
  // entries tq*NQ .. tq*NQ+NQ-1 of token row tr, group g
  const uint32_t vb = (uint32_t)(tr * bc_row + (g * k.N + tq * NQ) * ES);

  float A2[NPL], h[NPL];
#pragma unroll
  for (int i = 0; i < NPL; ++i) {
    const int e = n + 16 * i;
    A2[i] = -expf(k.A_log[cc * k.N + e]) * kLog2e;
    h[i] = k.h0 ? k.h0[(b * k.Dc + cc) * k.N + e] : 0.0f;
  }
  for (int j = 0; j < s; ++j) {  // carry in from the slices before this one
    const int64_t base = (b * k.nslices + j) * k.Dc + cc;
    const float sdt = k.ws_sdt[base];
#pragma unroll
    for (int i = 0; i < NPL; ++i) h[i] = fmaf(fast_exp2(A2[i] * sdt), h[i], k.ws_h[base * k.N + n + 16 * i]);
  }
  const float bias = k.dt_bias[cc];
  const float Dv = k.D[cc];
  const float inv_n = 1.0f / (float)k.N;
  const bool bc_norm = k.bc_eps > 0.0f;

  // a thread's pieces: token rows tr + 64 r of the tile (r < RT)
  auto rowo = [&](uint32_t o, int r, uint32_t row) { return o == kOOB ? kOOB : o + (uint32_t)(64 * r) * row; };
  struct Raw {
    RawVec<WA> x[RT], d[RT], z[RT];
    RawVec<WQ> bq[RT], cq[RT];
  };
  auto load_raw = [&](Raw& r, int t0) {
    const __amdgpu_buffer_rsrc_t rx = tile_rsrc(xb, t0, row_bytes), rd = tile_rsrc(db, t0, row_bytes);
    const __amdgpu_buffer_rsrc_t rz = tile_rsrc(zb, t0, row_bytes);
    const __amdgpu_buffer_rsrc_t rB = tile_rsrc(Bb, t0, bc_row), rC = tile_rsrc(Cb, t0, bc_row);
#pragma unroll
    for (int q = 0; q < RT; ++q) {
      r.x[q].load(rx, rowo(vx, q, row_bytes));
      r.d[q].load(rd, rowo(vx, q, row_bytes));
      if (GATE) r.z[q].load(rz, rowo(vx, q, row_bytes));
      r.bq[q].load(rB, rowo(vb, q, bc_row));
      r.cq[q].load(rC, rowo(vb, q, bc_row));
    }
  };
  // 4 activations as loaded into LDS (8 bytes of bf16 or 16 of fp32)
  auto put4 = [&](T* dst, RawVec<WA>& v) {
    if constexpr (ES == 2) {
      *reinterpret_cast<u32x2*>(dst) = u32x2{v.w[0], v.w[1]};
    } else {
      *reinterpret_cast<u32x4*>(dst) = u32x4{v.w[0], v.w[1], v.w[2], v.w[3]};
    }
  };
  auto stage = [&](Raw& r) {
#pragma unroll
    for (int q = 0; q < RT; ++q) {
      const int row = tr + 64 * q;
      put4(&sX[0][row][4 * tq], r.x[q]);
      put4(&sX[1][row][4 * tq], r.d[q]);
      if (GATE) put4(&sX[2][row][4 * tq], r.z[q]);
      float bv[NQ], cv[NQ];
      r.bq[q].template unpack<T>(bv);
      r.cq[q].template unpack<T>(cv);
      if (bc_norm) {  // uniform: the weightless RMS norm of B and C over the state entries
        float sb = 0.0f, sc = 0.0f;
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
      for (int j = 0; j < NQ; ++j) {
        sBC[0][tq * NQ + j][row] = bv[j];
        sBC[1][tq * NQ + j][row] = cv[j];
      }
    }
  };
  // y of the tile from t0 (complete in sY, in the output dtype) to memory: 4 channels
  // of a token row per thread and row.
  auto store_y = [&](int t0) {
    const __amdgpu_buffer_rsrc_t ry = tile_rsrc(yb, t0, row_bytes);
#pragma unroll
    for (int q = 0; q < RT; ++q) {
      const T* src = &sY[tr + 64 * q][4 * tq];
      if constexpr (ES == 2) {
        __builtin_amdgcn_raw_buffer_store_b64(*reinterpret_cast<const u32x2*>(src), ry, (int)rowo(vx, q, row_bytes), 0,
                                              0);
      } else {
        __builtin_amdgcn_raw_buffer_store_b128(*reinterpret_cast<const u32x4*>(src), ry, (int)rowo(vx, q, row_bytes),
                                               0, 0);
      }
    }
  };

  // Group j (tokens t0+16j .. t0+16j+15) of the tile in LDS. TAIL: the tile may
  // run past the slice's end (only the last tile does), so its steps are masked.
  auto compute_group = [&](int t0, int j, auto tail) {
    constexpr bool TAIL = decltype(tail)::value;
    const int tg = t0 + 16 * j;
    const int tl = 16 * j + n;  // this lane's token in the tile
    f32x4 b4[4][NPL], c4[4][NPL];  // B and C of the group's 16 tokens, this lane's entries
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4)
#pragma unroll
      for (int i = 0; i < NPL; ++i) {
        b4[q4][i] = *reinterpret_cast<const f32x4*>(&sBC[0][n + 16 * i][16 * j + 4 * q4]);
        c4[q4][i] = *reinterpret_cast<const f32x4*>(&sBC[1][n + 16 * i][16 * j + 4 * q4]);
      }
    const float xv = quad::to_f<T>(sX[0][tl][cl]);
    const float sp = softplus_fast(quad::to_f<T>(sX[1][tl][cl]) + bias);
    const float dtv = (!TAIL || tg + n < t_end) ? sp : 0.0f;  // a token past the end is a zero step
    const float dtx = dtv * xv;
    float p[16];
    static_for<16>([&](auto S) {
      constexpr int st = decltype(S)::value;
      const float dk = row_bcast<st>(dtv);
      const float xk = row_bcast<st>(dtx);
      float acc = 0.0f;
#pragma unroll
      for (int i = 0; i < NPL; ++i) {
        const float bv = b4[st / 4][i][st % 4], cv = c4[st / 4][i][st % 4];
        h[i] = fmaf(fast_exp2(dk * A2[i]), h[i], xk * bv);
        acc = i == 0 ? cv * h[i] : fmaf(cv, h[i], acc);
      }
      p[st] = acc;
      if (STATES) {
        const int tk = tg + st;
        if (tk < t_end && active) {
          float* sp_ = k.states + ((b * k.L + tk) * k.Dc + c) * k.N;
#pragma unroll
          for (int i = 0; i < NPL; ++i) sp_[n + 16 * i] = h[i];
        }
      }
    });
    float yv = row_transpose_sum_banked(p, n) + Dv * xv;
    if (GATE) yv *= silu(quad::to_f<T>(sX[2][tl][cl]));
    sY[tl][cl] = quad::from_f<T>(yv);
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
#pragma unroll
      for (int j = 0; j < TILE / 16; ++j) compute_group(t0, j, std::false_type{});
    } else {
#pragma unroll
      for (int j = 0; j < TILE / 16; ++j) compute_group(t0, j, std::true_type{});
    }
  }
  __syncthreads();
  if (t_end > t_begin) store_y(t_begin + ((t_end - t_begin - 1) / TILE) * TILE);

  if (s == k.nslices - 1 && active) {
#pragma unroll
    for (int i = 0; i < NPL; ++i) k.h_out[(b * k.Dc + c) * k.N + n + 16 * i] = h[i];
  }
}

template <typename T, int NP>
void launch_m1_row_np(const M1F& k, bool gate, bool states, dim3 grid, size_t dyn_lds, hipStream_t s) {
  const dim3 blk(256);
  if (gate && states) hipLaunchKernelGGL((m1_row_kernel<T, NP, true, true>), grid, blk, dyn_lds, s, k);
  else if (gate) hipLaunchKernelGGL((m1_row_kernel<T, NP, true, false>), grid, blk, dyn_lds, s, k);
  else if (states) hipLaunchKernelGGL((m1_row_kernel<T, NP, false, true>), grid, blk, dyn_lds, s, k);
  else hipLaunchKernelGGL((m1_row_kernel<T, NP, false, false>), grid, blk, dyn_lds, s, k);
}

}  // namespace sscan
