// ssd_chunk.hip -- the Mamba-2 SSD prompt scan on MFMA for gfx950 (bf16 or fp32 in, fp32 state;
// the fp32 kernel is described at ssd_chunk_f32_kernel below).
//
// What it computes ("Mamba-2", nnterp encyclopedia, sections "The mixer's
// values", "The hidden attention", "The state" and "The block, in order"):
// per head h, with dt_t = softplus(dt_raw[t, h] + dt_bias[h]) and
// a_t = dt_t * A_h (A_h = -exp(A_log[h])), the state S [head_dim, state_dim]
// follows S_t = exp(a_t) S_{t-1} + dt_t x_t B_t^T and y_t = S_t C_t + D_h x_t,
// then y * silu(z). Equivalently, inside a run of tokens from a known entering
// state S_in, with cs_t the cumulative sum of a from the start of the run,
//     y_i = sum_{j<=i} (C_i . B_j) exp(cs_i - cs_j) dt_j x_j      (the pages'
//           masked "hidden attention" restricted to the run)
//         + exp(cs_i) S_in C_i + D_h x_i,
//     S_out = exp(cs_last) S_in + sum_j exp(cs_last - cs_j) dt_j x_j B_j^T.
// This kernel applies those two identities to consecutive chunks of Q = 64
// tokens, carrying the state from chunk to chunk. Both are exact restatements
// of the recurrence; only rounding differs.
//
// Mapping: persistent workgroups of 4 waves, one per compute unit, take work
// items from per-die queues; an item is a segment of consecutive chunks of one
// chain (a head of a batch row), and segments of a chain hand the state on
// through the workspace (see the notes at state_in / state_out and ssd_plan).
// Within an item the chunks are walked in order. Wave w owns head_dim columns
// [16w, 16w+16): its slice of the state lives in fp32 MFMA accumulators (8 tiles
// of 16x16, state_dim 128) for the whole item. The output is computed
// transposed, Y^T = X^T M^T + S C^T, so that each lane ends up holding 4
// neighbouring head_dim columns of one token row; y then leaves through LDS as
// whole rows.
//
// G = C B^T of a chunk is the same for every head of a group, so ssd_cb_kernel
// computes it once per (batch row, chunk, group) before the scan: the ten
// lower-triangular 16x16 tiles, fp32, in the layout of the MFMA result (see
// there). The scan's waves load the tiles they mask one chunk ahead.
//
// Per chunk, between two barriers:
//   after barrier A (chunk staged in LDS: B and x row-major, C in the k order of
//   the S C^T operand, cumulative decay):
//     - x^T fragments and the epilogue's x values move from LDS to registers;
//     - the chunk's G tiles (10 over the 4 waves) are masked and scaled into
//       M[i, j] = G[i, j] exp(cs_i - cs_j) dt_j (bf16, LDS);
//     - Y^T = S_in C^T (A operand straight from the state accumulators), columns
//       scaled by exp(cs_i);
//     - S = exp(cs_last) S + B^T (w x), w_j = exp(cs_last - cs_j) dt_j, with the
//       B^T and x^T operands read from row-major LDS by the gfx950 transposing
//       LDS load (ds_read_b64_tr_b16);
//   after barrier B (M complete; every other LDS read of the chunk is done):
//     - Y^T += X^T M^T, then y = (Y + D x) silu(z) stored as 8-byte row pieces;
//     - the next chunk is staged into LDS from the registers its loads filled.
// The next chunk's loads are issued in parts between the phases above.
// All global traffic goes through buffer resources based at the chunk's first
// token row and ending at the sequence end, so rows past the end read zeros and
// drop their stores in hardware, with uniform offsets (no per-lane scalar offset).
//
// MFMA: v_mfma_f32_16x16x32_bf16. Operand layouts (verified on gfx950):
// A[16 x 32]: lane l holds row l%16, 8 values of k for lane group g = l/16;
// B[32 x 16]: lane l holds column l%16, the same k; D[16 x 16]: lane l holds rows
// 4g + r (r = 0..3), column l%16. Any assignment of k to (lane group, element)
// works as long as A and B use the same one.
// Transposing LDS load (verified on gfx950): within each 16-lane group, lanes
// 4q..4q+3 supply the addresses of 4 consecutive bf16 each (columns c0 + 4(a%4))
// of tile row q, and lane i receives tile rows 0..3 of column c0 + i. The LDS
// serves these loads 32 lanes at a time, so the two 16-lane groups of a half
// wave must hit disjoint banks: with the row pitches here that holds when tile
// row q is LDS row k0 + 2q (k0 + 2q + 1 for the second load), and not for
// consecutive rows. So within each 8 tokens k0..k0+7 the MFMA k order is
// 0, 2, 4, 6, 1, 3, 5, 7 (kperm); the other operands follow it: w is stored in
// that order and the masked M with its columns permuted the same way.
#include <math.h>

#include <algorithm>

#include "device_common.hpp"
#include "launch.hpp"

namespace sscan {

namespace {

constexpr int Q = 64;        // tokens per chunk
constexpr int P = 64;        // head_dim
constexpr int NS = 128;      // state_dim
constexpr int LDB = NS + 24;  // row pitch (bf16) of sB: 76 dwords = 12 mod 64, so the 4-row
                              // windows of the transposing loads hit distinct banks
constexpr int LDC = NS + 16;  // row pitch of sCk: 72 dwords, where 16-byte reads of
                              // 16 rows (the MFMA operands) are conflict-free
constexpr int kTiles = 10;    // lower-triangular 16x16 tiles of a chunk's C B^T
constexpr int kTileFloats = 256;  // one tile: 64 lanes x 4 fp32
constexpr int LDX = P + 8;   // row pitch of sX
constexpr int LDM = Q + 8;   // row pitch of sM
constexpr size_t kCkBytes = (size_t)Q * LDC * 2;
// The wave that computes the chunk's steps and decays while staging: one of the
// two waves whose third G tile is a repeat (waves 0 and 1 mask three tiles).
constexpr int kDecayWave = 3;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));

// E: the activations' element type (bf16 bits for ssd_chunk_kernel, float for
// ssd_chunk_f32_kernel)
template <typename E>
struct SsdKT {
  const E* x;
  const E* dt;
  const float* dt_bias;
  const float* A_log;
  const E* B;
  const E* C;
  const float* D;
  const E* z;
  const float* cb;  // C B^T tiles from ssd_cb_kernel: [batch, nchunks, G][10 tiles][64 lanes][4]
  const float* h0;
  E* y;
  float* h_out;
  unsigned* queue;  // [16 q]: next item of queue q; [128]: a wait gave up; [256 + ch]: segments of chain ch done
  float* carry;     // [batch * H, P, NS]: the state a segment hands to the next one, per head
  // H counts heads of P = 64 columns: a caller's head of 64 * 2^hshift columns is
  // 2^hshift of them, which share that head's step, decay and D (dt_raw has H >> hshift
  // columns; dt_bias, A_log and D H >> hshift entries)
  int64_t L, H, G;
  int nchunks;      // chunks of 64 tokens per batch row (ceil(L / 64))
  int heads_per_group;
  int nchains;      // batch * H / HPW (a chain is a run of HPW heads of one batch row)
  int seg_chunks;   // chunks per segment
  int nseg;         // segments per chain
  int nq;           // work queues; workgroup i serves queue i % nq, which holds chains
                    // [q nchains / nq, (q + 1) nchains / nq): item i of a queue with n chains is
                    // segment i / n of its chain i % n
  int hshift;       // log2(caller's head_dim / 64)
  // two passes (kLocal, then kFolded): lam[s * nstates + head] is the sum over segment s
  // of the head's a_t (exp2 domain), carry[s * nstates + head] its state from zero
  float* lam;
  int nstates;      // batch * H
};
typedef SsdKT<uint16_t> SsdK;
typedef SsdKT<float> SsdKF;

// Tile ti of a chunk's lower triangle -> (row block It, column block Jt), It >= Jt:
// (0,0) (1,0) (2,0) (3,0) (1,1) (2,1) (3,1) (2,2) (3,2) (3,3)
__device__ __forceinline__ int tile_j(int ti) { return ti < 4 ? 0 : (ti < 7 ? 1 : (ti < 9 ? 2 : 3)); }
__device__ __forceinline__ int tile_i(int ti) { return ti < 4 ? ti : (ti < 7 ? ti - 3 : (ti < 9 ? ti - 5 : 3)); }

// Position of token t of a chunk in k order (see the note on the transposing load):
// within each group of 8, token 8g + t sits at 8g + (t even ? t/2 : 4 + t/2).
__device__ __forceinline__ int kslot(int t) { return (t & ~7) | ((t & 1) << 2) | ((t & 7) >> 1); }

typedef __attribute__((address_space(4))) const SsdK KArgs;
typedef __attribute__((address_space(4))) const SsdKF KArgsF;
// The kernel's arguments, read again from the argument segment: used where a
// value is needed rarely, so that it does not hold a scalar register.
__device__ __forceinline__ KArgs* kargs() {
  uint64_t v = (uint64_t)__builtin_amdgcn_kernarg_segment_ptr();
  asm volatile("" : "+s"(v));
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v), hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (KArgs*)(((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ KArgsF* kargs_f() { return (KArgsF*)kargs(); }

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ u32x4 lds128(const uint16_t* p) { return *(const u32x4*)p; }
__device__ __forceinline__ u32x2 lds64(const uint16_t* p) { return *(const u32x2*)p; }

// 4 bf16 through the transposing LDS load (see the layout note above).
__device__ __forceinline__ u32x2 lds_tr(const uint16_t* p) {
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
  return __builtin_bit_cast(u32x2, v);
}

// two floats to two bf16 (round to nearest even, v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  const bf16x2 v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ float lo_f(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_f(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Cache policy of a buffer access that is coherent across the compute dies
// (sc1 on gfx950: written through to memory, read from the coherent level).
constexpr int kDeviceCoherent = 16;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, uint64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)(uint32_t)bytes, 0x00020000);
}

// Inclusive prefix sum over the 64 lanes of a wave with DPP: Hillis-Steele
// shifts within each row of 16 lanes, then the last lane of row 0 (row 2) is
// added to row 1 (row 3), and lane 31 to rows 2 and 3.
#define SSCAN_DPP(x, ctrl, rmask) \
  __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), (ctrl), (rmask), 0xF, false))
__device__ __forceinline__ float wave_inclusive_sum(float x) {
  x += SSCAN_DPP(x, 0x111, 0xF);  // row_shr:1
  x += SSCAN_DPP(x, 0x112, 0xF);  // row_shr:2
  x += SSCAN_DPP(x, 0x114, 0xF);  // row_shr:4
  x += SSCAN_DPP(x, 0x118, 0xF);  // row_shr:8
  x += SSCAN_DPP(x, 0x142, 0xA);  // row_bcast:15 into rows 1 and 3
  x += SSCAN_DPP(x, 0x143, 0xC);  // row_bcast:31 into rows 2 and 3
  return x;
}

// One pass: the entering state of the current item: the caller's (or zeros) for a first
// segment, else the one the previous segment left in carry, once its chain's
// flag says so. The producer of that segment holds an item dequeued earlier
// than this one, so it is running and never waits on this workgroup: the wait
// ends. Its bound (2^20 polls, about a second) only guarantees that the kernel
// terminates; a wait that gives up raises queue[128], which ends every other
// wait, and starts its item from a NaN state: every output that depends on a
// hand-off that did not happen (the rest of that chain's y and its final
// state) comes out NaN rather than silently wrong.
// carry and the flags move through device-coherent loads and stores (the sc1
// cache policy, as device-scope atomics use), which need no cache write-back
// or invalidation (either would flush the L2 that the other workgroups share);
// carry moves in 16-byte pieces, so the write-through goes out in whole
// 64-byte segments.
// (Both chunk kernels: the fields used here sit at the same offsets in SsdK and SsdKF.)
// hacc: this wave's state slice, S[p = 16 wq + li][n = 16 nt + 4 lg + r] in lane l,
// register r of tile nt; flag_ix: the chain's flag; state_ix: the head's state; s_lane:
// the lane's offset in a [P, NS] state; ticket: a word of workgroup memory.
__device__ __forceinline__ void chain_state_in_chained(f32x4 (&hacc)[8], int tid, int seg, int64_t flag_ix,
                                                       int64_t state_ix, int64_t s_lane, int& ticket) {
  if (seg > 0) {
    if (tid == 0) {
      unsigned* flag = kargs()->queue + 256 + flag_ix;
      bool ready = false, quit = false;
      for (int n = 0; n < (1 << 20) && !ready && !quit; ++n) {
        ready = __hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= (unsigned)seg;
        quit = !ready && __hip_atomic_load(kargs()->queue + 128, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0u;
        if (!ready && !quit) __builtin_amdgcn_s_sleep(2);
      }
      if (!ready) __hip_atomic_store(kargs()->queue + 128, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      ticket = ready ? 0 : 1;
    }
    __syncthreads();
    if (__builtin_amdgcn_readfirstlane(ticket) != 0) {
#pragma unroll
      for (int nt = 0; nt < 8; ++nt) hacc[nt] = f32x4{NAN, NAN, NAN, NAN};
    } else {
      const __amdgpu_buffer_rsrc_t rS = rsrc(kargs()->carry + state_ix * (P * NS), P * NS * 4);
#pragma unroll
      for (int nt = 0; nt < 8; ++nt)
        hacc[nt] = __builtin_bit_cast(
            f32x4, __builtin_amdgcn_raw_buffer_load_b128(rS, (int)((s_lane + 16 * nt) * 4), 0, kDeviceCoherent));
    }
  } else if (kargs()->h0) {
    const float* src = kargs()->h0 + state_ix * (P * NS) + s_lane;
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) hacc[nt] = *(const f32x4*)(src + 16 * nt);
  } else {
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) hacc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
}

// The entering state of segment seg in the second of two passes: h0 (or zeros) for
// the first segment, else carry[seg - 1], where ssd_fold_states_kernel left S_in(seg)
// (plain loads: it was an earlier kernel).
__device__ __forceinline__ void chain_state_in_folded(f32x4 (&hacc)[8], int seg, int64_t state_ix, int64_t s_lane) {
  const float* src = seg > 0 ? kargs()->carry + ((int64_t)(seg - 1) * kargs()->nstates + state_ix) * (P * NS)
                             : kargs()->h0 ? kargs()->h0 + state_ix * (P * NS) : nullptr;
  if (src) {
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) hacc[nt] = *(const f32x4*)(src + s_lane + 16 * nt);
  } else {
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) hacc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
}

// Between the two passes: the first left each segment j's state from zero, L_j, in
// carry[j] and its decay sum lam_j (exp2 domain). S_in(0) = h0 (or zeros) and
// S_in(j + 1) = 2^lam_j S_in(j) + L_j, the recurrence restated at segment ends; each
// carry[j] is replaced by S_in(j + 1). One thread per 4 entries of a state, a step per
// segment; four segments' loads are issued before their updates.
__global__ __launch_bounds__(256) void ssd_fold_states_kernel(float* __restrict__ carry, const float* __restrict__ lam,
                                                              const float* __restrict__ h0, int nstates, int nfold) {
  constexpr int64_t per = P * NS / 4;  // threads per state
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= nstates * per) return;
  const int64_t st = i / per, e = (i % per) * 4;
  const int64_t stride = (int64_t)nstates * (P * NS);  // from segment j to j + 1
  float* base = carry + st * (P * NS) + e;
  f32x4 s = h0 ? *(const f32x4*)(h0 + st * (P * NS) + e) : f32x4{0.f, 0.f, 0.f, 0.f};
  for (int j = 0; j < nfold; j += 4) {
    f32x4 v[4];
    float d[4];
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (j + u < nfold) {
        v[u] = *(const f32x4*)(base + (j + u) * stride);
        d[u] = fast_exp2(lam[(int64_t)(j + u) * nstates + st]);
      }
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (j + u < nfold) {
#pragma unroll
        for (int r = 0; r < 4; ++r) s[r] = fmaf(d[u], s[r], v[u][r]);
        *(f32x4*)(base + (j + u) * stride) = s;
      }
  }
}

// Work modes of the chunk kernels. kChained: one pass, a segment waits for its
// predecessor's state (chain_state_in_chained). Two passes for few chains, where
// the segments of a chain can then run at once: kLocal computes each segment but
// the last from a zero state, only the state update (no y), and leaves that state
// and the segment's decay sum; ssd_fold_states_kernel turns those into the segments'
// entering states; kFolded then runs every segment from its entering state
// (chain_state_in_folded), with no waits.
constexpr int kChained = 0, kLocal = 1, kFolded = 2;

template <int MODE>
__device__ __forceinline__ void chain_state_in(f32x4 (&hacc)[8], int tid, int seg, int64_t flag_ix, int64_t state_ix,
                                               int64_t s_lane, int& ticket) {
  if constexpr (MODE == kLocal) {
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) hacc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
    return;
  } else if constexpr (MODE == kFolded) {
    chain_state_in_folded(hacc, seg, state_ix, s_lane);
  } else {
    chain_state_in_chained(hacc, tid, seg, flag_ix, state_ix, s_lane, ticket);
  }
  // The loads complete here: otherwise every chunk would wait for them (and
  // for the chunk loads queued behind them) before it first reads the state.
#pragma unroll
  for (int nt = 0; nt < 8; ++nt) asm volatile("" : "+v"(hacc[nt]));
}

// The leaving state. kChained: to the caller after the last segment, else to carry
// and then the chain's flag (every thread waits until its stores are complete,
// visible to the device, before the barrier; thread 0 raises the flag after it).
// kFolded: to the caller after the last segment (the others' went to carry in the
// first pass). kLocal: to carry[seg], with the decay sum lam (one head per workgroup).
template <int MODE>
__device__ __forceinline__ void chain_state_out(const f32x4 (&hacc)[8], int tid, int seg, int64_t flag_ix,
                                                int64_t state_ix, int64_t s_lane, float lam = 0.0f) {
  if constexpr (MODE == kLocal) {
    const int64_t nst = kargs()->nstates;
    float* dst = kargs()->carry + (seg * nst + state_ix) * (P * NS) + s_lane;
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) *(f32x4*)(dst + 16 * nt) = hacc[nt];
    if (tid == 0) kargs()->lam[seg * nst + state_ix] = lam;
  } else if (MODE == kChained && seg + 1 < kargs()->nseg) {
    const __amdgpu_buffer_rsrc_t rS = rsrc(kargs()->carry + state_ix * (P * NS), P * NS * 4);
#pragma unroll
    for (int nt = 0; nt < 8; ++nt)
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, hacc[nt]), rS, (int)((s_lane + 16 * nt) * 4), 0,
                                             kDeviceCoherent);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the stores above have completed
    __syncthreads();
    if (tid == 0) __hip_atomic_store(kargs()->queue + 256 + flag_ix, (unsigned)(seg + 1), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  } else if (MODE == kChained || seg + 1 == kargs()->nseg) {
    float* dst = kargs()->h_out + state_ix * (P * NS) + s_lane;
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) *(f32x4*)(dst + 16 * nt) = hacc[nt];
  }
}

// One chunk's staged global loads of one thread, in flight during the previous
// chunk. Coalesced: 16 lanes cover a 256-byte row of B or C (an instruction, 4
// rows), 8 lanes a 128-byte row of x (8 rows), so each load touches a few cache
// lines rather than one per lane. B, C (shared by the workgroup's heads): rows
// tid/16 + 16 HPW it, piece tid%16; x and z (per head): rows 16wq + 8it + l/8,
// piece l%8; dt (wave kDecayWave of each head only): token l.
template <int HPW>
struct Prefetch {
  u32x4 b[4 / HPW], c[4 / HPW], x[2], z[2];
  f32x4 g[HPW == 1 ? 3 : 2];  // the C B^T tiles this wave masks
  uint32_t dt;  // raw bf16 bits
};

}  // namespace

// HPW heads of one batch row per workgroup (1 or 2), four waves per head. With two
// heads, B and C (shared by every head of a group) are staged once and each C B^T
// tile is loaded once, then masked with each head's decays; the two heads' waves
// share the SIMDs, so one head's MFMA and memory latencies hide behind the other's
// work.
// SPLIT: the state as C reads it and the weighted inputs w x that update it are each
// carried as two bf16 parts (hi = RNE(v), lo = RNE(v - hi)), about 16 significant bits
// instead of 8, at twice the MFMAs of those two products (the precise form, on request).
template <int HPW, int MODE, bool SPLIT = false>
__global__ __launch_bounds__(256 * HPW, HPW == 1 ? 2 : 1) void ssd_chunk_kernel(SsdK k) {
  static_assert(MODE == kChained || HPW == 1, "two passes: one head per workgroup");
  static_assert(!SPLIT || HPW == 1, "the precise form: one head per workgroup");
  constexpr bool Y = MODE != kLocal;  // the pass computes y (kLocal: only the state)
  constexpr int NW = 4 * HPW;      // waves
  constexpr int BCIT = 4 / HPW;    // rows of B (and of C) a thread stages
  constexpr int NT = HPW == 1 ? 3 : 2;  // C B^T tiles a wave masks (some repeated)
  __shared__ __attribute__((aligned(16))) uint16_t sB[Q * LDB];
  // C, each row in the k order of the Y^T = S C^T operand: positions
  // 32kb + 8lg + e hold states 32kb + 4lg + e (e < 4) and 32kb + 16 + 4lg + e - 4
  // (e >= 4), so that operand is one 16-byte read (the state accumulators fix
  // that order)
  // (dynamic LDS of kCkBytes: its size then does not lower the occupancy the code
  // is compiled for, which schedules this kernel better)
  extern __shared__ __attribute__((aligned(16))) uint16_t sCk[];
  __shared__ __attribute__((aligned(16))) uint16_t sX[HPW][Q * LDX];
  __shared__ __attribute__((aligned(16))) uint16_t sM[HPW][Q * LDM];
  __shared__ __attribute__((aligned(16))) uint16_t sZ[HPW][Q * LDX];  // z of the chunk
  __shared__ __attribute__((aligned(16))) uint16_t sY[HPW][Q * LDX];  // y of the chunk, stored after the next barrier
  __shared__ __attribute__((aligned(16))) float sCS[HPW][Q], sDT[HPW][Q], sW[HPW][Q], sE[HPW][Q];
  __shared__ int sTicket[3];  // [0]: the first item; [1]: the item after the current one;
                              // [2]: the current item's hand-off wait gave up

  // the wave index through readfirstlane: a scalar, so branches on it stay uniform;
  // wave w serves head slot hs = w / 4 of the workgroup's heads, columns 16 wq .. 16 wq + 15
  const int tid = threadIdx.x, w = __builtin_amdgcn_readfirstlane(tid >> 6), hs = w >> 2, wq = w & 3,
            l = tid & 63, li = l & 15, lg = l >> 4;
  // 32-bit sizes: the host guarantees each batch row of every tensor is < 2^31 bytes
  const int L = (int)k.L, H = (int)k.H, G = (int)k.G;
  const int hpc = H / HPW;  // chains (runs of HPW heads) per batch row
  const bool gate = k.z != nullptr;

  // This workgroup's queue (the dispatcher deals workgroups to the eight compute
  // dies in turn, so the queues match the dies and a die's L2 serves neighbouring
  // heads, which share B and C): its counter, first chain, chains and items.
  // Computed where needed from the argument segment, so that none holds a
  // scalar register through the chunk loop.
  // (32-bit: chains < 2^24 and queues <= 8; readfirstlane marks the quotients
  // uniform, so buffer resources built from them stay scalar)
  auto qindex = [&]() { return __builtin_amdgcn_readfirstlane((int)(blockIdx.x % (unsigned)kargs()->nq)); };
  // (kLocal: its own counters, in the words of the chain flags, which two passes do not use)
  auto qcounter = [&]() { return kargs()->queue + (MODE == kLocal ? 256 : 0) + 16 * qindex(); };
  auto qfirst = [&]() {
    return __builtin_amdgcn_readfirstlane((int)((unsigned)(qindex() * kargs()->nchains) / (unsigned)kargs()->nq));
  };
  auto qchains = [&]() {
    const unsigned q = (unsigned)qindex(), n = (unsigned)kargs()->nchains, nq = (unsigned)kargs()->nq;
    return __builtin_amdgcn_readfirstlane((int)((q + 1) * n / nq - q * n / nq));
  };
  // (kLocal: every segment but the last)
  auto qitems = [&]() { return (MODE == kLocal ? kargs()->nseg - 1 : kargs()->nseg) * qchains(); };

  // Work items come from a counter. Each workgroup takes its first item at
  // once and the second after its first chunk is staged (by then every
  // workgroup of the grid has taken its first, so the first round is items
  // 0 .. grid-1); after that it takes an item when it starts the last chunk of
  // the current one, so that it knows the next item one item ahead and can
  // load the next item's first chunk during the current item's last chunk.
  if (tid == 0) sTicket[0] = (int)atomicAdd(qcounter(), 1u);
  __syncthreads();
  int cur = __builtin_amdgcn_readfirstlane(sTicket[0]);
  if (cur >= qitems()) return;  // the whole workgroup
  int nxt = -1;

  // (dt_raw has one column per caller's head: H >> hshift)
  const int Hd = H >> k.hshift;
  const uint32_t bc_row = (uint32_t)(G * NS * 2), xz_row = (uint32_t)(H * P * 2), dt_row = (uint32_t)(Hd * 2);
  // elements per batch row
  const uint32_t bc_bat = (uint32_t)L * (G * NS), xz_bat = (uint32_t)L * (H * P), dt_bat = (uint32_t)L * Hd;
  const int bc_r = tid >> 4, bc_p = tid & 15;         // staging row (+ 16 HPW it) and piece of B, C
  const int x_r = 16 * wq + (l >> 3), x_p = l & 7;    // staging row (+ 8 it) and piece of x
  const uint32_t bc_lane = (uint32_t)(bc_r * bc_row + bc_p * 16);
  const uint32_t x_lane = (uint32_t)(x_r * xz_row + x_p * 16);
  const uint32_t dt_lane = (uint32_t)(l * dt_row);

  // Global access goes through buffer resources based at a chunk's first token
  // row and this wave's head's first column, ending at the sequence end (the host
  // guarantees each batch row is < 2^31 bytes): rows past the end read zeros and
  // drop their stores in hardware, and the lane offsets stay uniform.
  // Target of the loads in flight: batch row tb, this wave's head th, group tg,
  // first token tt (tt >= L: none; every load reads zeros).
  int tb = 0, th = 0, tg = 0, tt = 0;
  auto tgt_rsrc = [&](const uint16_t* base, uint32_t bat, uint32_t col, uint32_t rowb, bool on = true) {
    const int left = on ? L - tt : 0;
    return rsrc((const char*)(base + (uint64_t)tb * bat + col) + (uint32_t)tt * rowb,
                left > 0 ? (uint32_t)left * rowb - col * 2 : 0u);
  };
  auto load_b = [&](Prefetch<HPW>& pf) {
    const __amdgpu_buffer_rsrc_t rB = tgt_rsrc(k.B, bc_bat, (uint32_t)tg * NS, bc_row);
#pragma unroll
    for (int it = 0; it < BCIT; ++it)
      pf.b[it] = __builtin_amdgcn_raw_buffer_load_b128(rB, (int)(bc_lane + it * 16 * HPW * bc_row), 0, 0);
  };
  auto load_c = [&](Prefetch<HPW>& pf) {
    const __amdgpu_buffer_rsrc_t rC = tgt_rsrc(k.C, bc_bat, (uint32_t)tg * NS, bc_row);
#pragma unroll
    for (int it = 0; it < BCIT; ++it)
      pf.c[it] = __builtin_amdgcn_raw_buffer_load_b128(rC, (int)(bc_lane + it * 16 * HPW * bc_row), 0, 0);
  };
  // the target chunk's C B^T tiles that this wave masks (past the end: none)
  auto load_g = [&](Prefetch<HPW>& pf) {
    const float* blk = kargs()->cb + (((int64_t)tb * kargs()->nchunks + tt / Q) * G + tg) * (kTiles * kTileFloats);
    const __amdgpu_buffer_rsrc_t rG = rsrc(blk, tt < L ? kTiles * kTileFloats * 4 : 0u);
#pragma unroll
    for (int u = 0; u < NT; ++u) {
      const int ti = w + NW * u < kTiles ? w + NW * u : w;
      pf.g[u] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rG, (ti * 64 + l) * 16, 0, 0));
    }
  };
  auto load_x = [&](Prefetch<HPW>& pf) {
    const __amdgpu_buffer_rsrc_t rX = tgt_rsrc(k.x, xz_bat, (uint32_t)th * P, xz_row);
    // only the decay wave of a head uses dt: the other waves' resource is empty (no memory access)
    const __amdgpu_buffer_rsrc_t rD =
        tgt_rsrc(k.dt, dt_bat, (uint32_t)(th >> kargs()->hshift), dt_row, wq == kDecayWave);
#pragma unroll
    for (int it = 0; it < 2; ++it)
      pf.x[it] = __builtin_amdgcn_raw_buffer_load_b128(rX, (int)(x_lane + it * 8 * xz_row), 0, 0);
    pf.dt = __builtin_amdgcn_raw_buffer_load_b16(rD, (int)dt_lane, 0, 0);
  };
  // z of the target chunk, staged like x (without a gate: loads of x, unused)
  auto load_z = [&](Prefetch<HPW>& pf) {
    const __amdgpu_buffer_rsrc_t rZ = tgt_rsrc(gate ? k.z : k.x, xz_bat, (uint32_t)th * P, xz_row);
#pragma unroll
    for (int it = 0; it < 2; ++it)
      pf.z[it] = __builtin_amdgcn_raw_buffer_load_b128(rZ, (int)(x_lane + it * 8 * xz_row), 0, 0);
  };
  // y of the previous chunk: sY (written by the epilogue in its layout) to memory
  // as whole rows, through ry_prev (empty before the first chunk: no stores);
  // non-temporal (y is not read again here; measured about 1% faster)
  __amdgpu_buffer_rsrc_t ry_prev = rsrc(k.y, 0);
  auto store_y = [&]() {
#pragma unroll
    for (int it = 0; it < 2; ++it)
      __builtin_amdgcn_raw_buffer_store_b128(lds128(sY[hs] + (x_r + 8 * it) * LDX + x_p * 8), ry_prev,
                                             (int)(x_lane + it * 8 * xz_row), 0, 2);
  };

  // The current item: chain hc (heads hc HPW .. hc HPW + HPW - 1 of batch row b) and this
  // wave's head h of group g, chunks [c, c_end); per-head constants.
  int b = 0, hc = 0, h = 0, g = 0, c = 0, c_end = 0;
  int seg = 0;
  float A2 = 0.f, bias = 0.f, Dh = 0.f;
  auto set_item = [&](int it) {
    const KArgs* kk = kargs();
    const int nch = qchains();
    seg = it / nch;
    const int ch = qfirst() + it % nch;
    b = ch / hpc;
    hc = ch % hpc;
    h = hc * HPW + hs;
    g = h / kk->heads_per_group;  // the host guarantees the chain's heads share a group
    c = seg * kk->seg_chunks;
    c_end = min(c + kk->seg_chunks, max((L + Q - 1) / Q, 1));  // seqlen 0: one empty chunk
    const int hp = h >> kk->hshift;  // the caller's head
    A2 = -expf(kk->A_log[hp]) * kLog2e;  // decay per unit step, exp2 domain
    bias = kk->dt_bias[hp];
    Dh = kk->D[hp];
  };

  // Chunk at token tt from the prefetch registers into LDS; wave kDecayWave of each
  // head adds that head's steps, their inclusive cumulative sum (exp2 domain) and the
  // derived decays.
  auto stage = [&](Prefetch<HPW>& pf) {
#pragma unroll
    for (int it = 0; it < BCIT; ++it) {
      const int row = bc_r + 16 * HPW * it;
      *(u32x4*)(sB + row * LDB + bc_p * 8) = pf.b[it];
      // states 8 bc_p + e: piece q = bc_p % 4 of the 32 states 32kb.. (kb = bc_p / 4)
      // goes to positions 32kb + 16 (q % 2) + 4 (q / 2) and 8 further on
      const int pk = 32 * (bc_p >> 2) + 16 * (bc_p & 1) + 4 * ((bc_p >> 1) & 1);
      if constexpr (Y) {
        *(u32x2*)(sCk + row * LDC + pk) = u32x2{pf.c[it][0], pf.c[it][1]};
        *(u32x2*)(sCk + row * LDC + pk + 8) = u32x2{pf.c[it][2], pf.c[it][3]};
      }
    }
#pragma unroll
    for (int it = 0; it < 2; ++it) {
      *(u32x4*)(sX[hs] + (x_r + 8 * it) * LDX + x_p * 8) = pf.x[it];
      if constexpr (Y) *(u32x4*)(sZ[hs] + (x_r + 8 * it) * LDX + x_p * 8) = pf.z[it];
    }
    if (wq == kDecayWave) {
      const int nt_valid = max(0, min(Q, L - tt));
      const float dtv = l < nt_valid ? softplus(lo_f(pf.dt) + bias) : 0.0f;  // past the end: a zero step
      const float cs = wave_inclusive_sum(dtv * A2);
      const float cs_last = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(cs), 63));
      sDT[hs][l] = dtv;
      sCS[hs][l] = cs;
      sE[hs][l] = fast_exp2(cs);
      sW[hs][kslot(l)] = fast_exp2(cs_last - cs) * dtv;  // in k order
    }
  };

  // state slice: hacc[nt][r] = S[p = 16wq + li][n = 16nt + 4lg + r] of head h; stored as [b, h, p, n]
  f32x4 hacc[8];
  const int64_t s_lane = (int64_t)(16 * wq + li) * NS + 4 * lg;
  // the entering state of the current item and the leaving one (chain_state_in / _out)
  float lam = 0.0f;  // kLocal: the item's decay sum so far (exp2 domain)
  auto state_in = [&]() {
    chain_state_in<MODE>(hacc, tid, seg, (int64_t)b * hpc + hc, (int64_t)b * H + h, s_lane, sTicket[2]);
    lam = 0.0f;
  };
  auto state_out = [&]() {
    chain_state_out<MODE>(hacc, tid, seg, (int64_t)b * hpc + hc, (int64_t)b * H + h, s_lane, lam);
  };

  // the tiles of M above the diagonal block row stay zero
  for (int e = tid; e < HPW * Q * LDM; e += 256 * HPW) (&sM[0][0])[e] = 0;

  set_item(cur);
  tb = b; th = h; tg = g; tt = c * Q;
  Prefetch<HPW> pf;
  load_b(pf);
  if constexpr (Y) {
    load_c(pf);
    load_g(pf);
  }
  load_x(pf);
  if constexpr (Y) load_z(pf);
  stage(pf);
  state_in();
  if (tid == 0) sTicket[1] = (int)atomicAdd(qcounter(), 1u);
  __syncthreads();
  {
    const int t = __builtin_amdgcn_readfirstlane(sTicket[1]);
    nxt = t < qitems() ? t : -1;
  }

  for (;;) {
    const int t0 = c * Q;
    const bool last = c + 1 == c_end;
    // ---- after barrier A: chunk c is in LDS. Loads now go to the next chunk of
    // this item, or to the first chunk of the next item.
    int ticket = 0;
    if (!last) {
      tt = t0 + Q;
    } else if (nxt >= 0) {
      const int qn = qchains(), ns = nxt / qn, nch = qfirst() + nxt % qn;
      tb = nch / hpc;
      th = (nch % hpc) * HPW + hs;
      tg = th / kargs()->heads_per_group;
      tt = ns * kargs()->seg_chunks * Q;
      if (tid == 0) ticket = (int)atomicAdd(qcounter(), 1u);  // the item after that
    } else {
      tt = L;
    }
    if constexpr (Y) store_y();  // the previous chunk's y (sY complete since barrier A)
    load_b(pf);
    if constexpr (Y) load_z(pf);

    // x^T fragments (A operand of Y^T += X^T M^T; k = j = 32kb + 8lg + kperm(e)) by
    // two transposing loads each, and the epilogue's x values (8 bytes of row 16it + li)
    u32x4 xa[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int k0 = 32 * kb + 8 * lg;
      const u32x2 lo = lds_tr(sX[hs] + (k0 + 2 * (li >> 2)) * LDX + 16 * wq + 4 * (li & 3));
      const u32x2 hi = lds_tr(sX[hs] + (k0 + 1 + 2 * (li >> 2)) * LDX + 16 * wq + 4 * (li & 3));
      xa[kb] = u32x4{lo[0], lo[1], hi[0], hi[1]};
    }
    u32x2 xe[4], zkeep[4];
    if constexpr (Y) {
#pragma unroll
      for (int it = 0; it < 4; ++it) {
        xe[it] = lds64(sX[hs] + (16 * it + li) * LDX + 16 * wq + 4 * lg);
        zkeep[it] = lds64(sZ[hs] + (16 * it + li) * LDX + 16 * wq + 4 * lg);
      }
    }

    // ---- G tiles -> M (lower triangle), each masked with every head's decays:
    // wave w takes tiles w, w + NW, w + 2 NW. A wave with fewer tiles masks its
    // first tile again, writing the same values again (no branch in the phase).
    if constexpr (Y) {
      f32x4 acc[NT];
      int Jt[NT], It[NT];
#pragma unroll
      for (int u = 0; u < NT; ++u) {
        const int ti = w + NW * u < kTiles ? w + NW * u : w;
        Jt[u] = tile_j(ti);
        It[u] = tile_i(ti);
        acc[u] = pf.g[u];  // loaded during the previous chunk
      }
      float csi[HPW][NT];
      f32x4 csj[HPW][NT], dtj[HPW][NT];
#pragma unroll
      for (int hh = 0; hh < HPW; ++hh)
#pragma unroll
        for (int u = 0; u < NT; ++u) {
          csi[hh][u] = sCS[hh][16 * It[u] + li];
          csj[hh][u] = *(const f32x4*)(sCS[hh] + 16 * Jt[u] + 4 * lg);
          dtj[hh][u] = *(const f32x4*)(sDT[hh] + 16 * Jt[u] + 4 * lg);
        }
#pragma unroll
      for (int u = 0; u < NT; ++u) {
        // acc[r] = G[i][j], i = 16It + li, j = 16Jt + 4lg + r
        const int i = 16 * It[u] + li;
#pragma unroll
        for (int hh = 0; hh < HPW; ++hh) {
          float m[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int j = 16 * Jt[u] + 4 * lg + r;
            // computed for every lane and selected (the clamp keeps masked entries finite)
            const float v = acc[u][r] * fast_exp2(fminf(csi[hh][u] - csj[hh][u][r], 0.0f)) * dtj[hh][u][r];
            m[r] = j <= i ? v : 0.0f;
          }
          // columns in k order: j = 16Jt + 4lg + r sits at 16Jt + 8(lg/2) + kslot(4(lg%2) + r)
          uint16_t* row = sM[hh] + i * LDM + 16 * Jt[u] + 8 * (lg >> 1) + 2 * (lg & 1);
          *(uint32_t*)row = pack2(m[0], m[2]);
          *(uint32_t*)(row + 4) = pack2(m[1], m[3]);
        }
      }
    }

    if constexpr (Y) {
      load_c(pf);
      load_g(pf);
    }
    // ---- Y^T = S_in C^T, columns scaled by exp(cs_i). A operand: the state,
    // k = n in {32kb + 4lg + r} U {32kb + 16 + 4lg + r} (the accumulator layout);
    // B operand: C[i][n] for the same n, 16 bytes of row i of sCk.
    // the row scales and the state update's weights (no scheduling barrier after
    // these reads: with the C B^T tiles from the pre-pass, letting the scheduler mix
    // them and the mask's work into the MFMAs measured 2.5% faster)
    float ei[4];
#pragma unroll
    for (int it = 0; it < 4; ++it) ei[it] = sE[hs][16 * it + li];
    f32x4 wj[2][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      wj[kb][0] = *(const f32x4*)(sW[hs] + 32 * kb + 8 * lg);
      wj[kb][1] = *(const f32x4*)(sW[hs] + 32 * kb + 8 * lg + 4);
    }
    const float dec_last = sE[hs][Q - 1];
    if constexpr (!Y) lam += sCS[hs][Q - 1];
    f32x4 yacc[4];
#pragma unroll
    for (int it = 0; it < 4; ++it) yacc[it] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < (Y ? 4 : 0); ++kb) {
      u32x4 sv, sl;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float a0 = hacc[2 * kb + (q >> 1)][2 * (q & 1)], a1 = hacc[2 * kb + (q >> 1)][2 * (q & 1) + 1];
        sv[q] = pack2(a0, a1);
        if constexpr (SPLIT) sl[q] = pack2(a0 - lo_f(sv[q]), a1 - hi_f(sv[q]));  // what hi leaves out
      }
      const bf16x8 aop = as_bf16x8(sv);
#pragma unroll
      for (int it = 0; it < 4; ++it) {
        const bf16x8 cop = as_bf16x8(lds128(sCk + (16 * it + li) * LDC + 32 * kb + 8 * lg));
        yacc[it] = mfma(aop, cop, yacc[it]);
        if constexpr (SPLIT) yacc[it] = mfma(as_bf16x8(sl), cop, yacc[it]);
      }
    }
#pragma unroll
    for (int it = 0; it < 4; ++it) {
#pragma unroll
      for (int r = 0; r < 4; ++r) yacc[it][r] *= ei[it];
    }

    load_x(pf);
    // ---- S = exp(cs_last) S + B^T (w x). A operand: B^T rows n = 16nt + li, k = j
    // (transposing loads of B); B operand: w_j x[j][16wq + li] from the x^T fragments
    // (both in k order; sW holds w in k order).
    bf16x8 wxb[2], wxl[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const f32x4 w0 = wj[kb][0], w1 = wj[kb][1];
      const u32x4 v = xa[kb];
      const float p[8] = {lo_f(v[0]) * w0[0], hi_f(v[0]) * w0[1], lo_f(v[1]) * w0[2], hi_f(v[1]) * w0[3],
                          lo_f(v[2]) * w1[0], hi_f(v[2]) * w1[1], lo_f(v[3]) * w1[2], hi_f(v[3]) * w1[3]};
      u32x4 hv, lv;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        hv[q] = pack2(p[2 * q], p[2 * q + 1]);
        if constexpr (SPLIT) lv[q] = pack2(p[2 * q] - lo_f(hv[q]), p[2 * q + 1] - hi_f(hv[q]));
      }
      wxb[kb] = as_bf16x8(hv);
      if constexpr (SPLIT) wxl[kb] = as_bf16x8(lv);
    }
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) {
#pragma unroll
      for (int r = 0; r < 4; ++r) hacc[nt][r] *= dec_last;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const int k0 = 32 * kb + 8 * lg;
        const u32x2 lo = lds_tr(sB + (k0 + 2 * (li >> 2)) * LDB + 16 * nt + 4 * (li & 3));
        const u32x2 hi = lds_tr(sB + (k0 + 1 + 2 * (li >> 2)) * LDB + 16 * nt + 4 * (li & 3));
        const bf16x8 bop = as_bf16x8(u32x4{lo[0], lo[1], hi[0], hi[1]});
        hacc[nt] = mfma(bop, wxb[kb], hacc[nt]);
        if constexpr (SPLIT) hacc[nt] = mfma(bop, wxl[kb], hacc[nt]);
      }
    }

    __syncthreads();  // ---- barrier B: M complete; no wave reads sB, sCk, sX or the decays again

    // ---- Y^T += X^T M^T (M[i][j] = 0 for j > i: skip the upper blocks)
#pragma unroll
    for (int it = 0; it < (Y ? 4 : 0); ++it) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        if (kb == 1 && it < 2) continue;
        const bf16x8 mb = as_bf16x8(lds128(sM[hs] + (16 * it + li) * LDM + 32 * kb + 8 * lg));
        yacc[it] = mfma(as_bf16x8(xa[kb]), mb, yacc[it]);
      }
    }
    // ---- epilogue: lane holds y[i = 16it + li][16wq + 4lg + r]; y = (Y + D x) silu(z)
    if constexpr (Y) {
      const __amdgpu_buffer_rsrc_t rY = rsrc((const char*)(k.y + (uint64_t)b * xz_bat + h * P) + (uint32_t)t0 * xz_row,
                                             (uint32_t)(L - t0) * xz_row - h * P * 2);
#pragma unroll
      for (int it = 0; it < 4; ++it) {
        const float xs[4] = {lo_f(xe[it][0]), hi_f(xe[it][0]), lo_f(xe[it][1]), hi_f(xe[it][1])};
        const float zs[4] = {lo_f(zkeep[it][0]), hi_f(zkeep[it][0]), lo_f(zkeep[it][1]), hi_f(zkeep[it][1])};
        float v[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) v[r] = fmaf(Dh, xs[r], yacc[it][r]) * (gate ? silu(zs[r]) : 1.0f);
        *(u32x2*)(sY[hs] + (16 * it + li) * LDX + 16 * wq + 4 * lg) = u32x2{pack2(v[0], v[1]), pack2(v[2], v[3])};
      }
      ry_prev = rY;
    }
    const bool finished = last && nxt < 0;
    if (last) {
      // ---- the item is done: hand its state on and switch to the next item
      state_out();
      if (!finished) {
        if (tid == 0) sTicket[1] = ticket;
        set_item(nxt);
        state_in();
        __syncthreads();  // sTicket[1]
        const int t = __builtin_amdgcn_readfirstlane(sTicket[1]);
        nxt = t < qitems() ? t : -1;
      }
    } else {
      ++c;
    }
    // ---- the next chunk into LDS (past the end, or after the last item: zeros,
    // harmless). The loop leaves only here, so every path back to its head passes
    // the waits of the staging: otherwise the next chunk would wait for this
    // chunk's stores.
    stage(pf);
    __syncthreads();  // ---- barrier A of the next chunk
    if (finished) break;
  }
  if constexpr (Y) store_y();  // the last chunk's y
}

// G = C B^T of every chunk of 64 tokens and every group, once for all the heads
// of the group (the scan's masked "hidden attention" inside a chunk, "Mamba-2",
// section "The hidden attention", before the per-head decays): the ten
// lower-triangular 16x16 tiles in the layout of the MFMA result, so that a lane of
// the scan reads its four values of a tile as one 16-byte piece:
//   cb[blk][ti][l][r] = sum_n C[t0 + 16 It + l % 16][n] B[t0 + 16 Jt + 4 (l / 16) + r][n],
// blk = (b nchunks + c) G + g, t0 = 64 c, (It, Jt) = the tile's blocks. Rows past
// the sequence end read zeros. One workgroup of 10 waves per block, one tile each.
// It also clears the scan's work queues, give-up word and chain flags (q, nq words;
// give_up != 0 raises the give-up word instead, the test of what a wait that gives
// up does): a kernel rather than a memset, so that the call can be captured in a
// graph, and this one rather than a kernel of its own, to save a launch.
__global__ __launch_bounds__(640) void ssd_cb_kernel(const uint16_t* __restrict__ B, const uint16_t* __restrict__ C,
                                                     float* __restrict__ cb, int L, int G, int nchunks, int64_t nblk,
                                                     unsigned* __restrict__ q, int nq, unsigned give_up) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < nq; i += gridDim.x * blockDim.x)
    q[i] = i == 128 ? give_up : 0u;
  const int ti = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)), l = threadIdx.x & 63, li = l & 15,
            lg = l >> 4;
  const uint32_t row = (uint32_t)(G * NS * 2);
  for (int64_t blk = blockIdx.x; blk < nblk; blk += gridDim.x) {
    const int g = (int)(blk % G), c = (int)((blk / G) % nchunks);
    const int64_t b = blk / ((int64_t)G * nchunks);
    const int t0 = c * Q;
    const uint32_t bytes = (uint32_t)(L - t0) * row - (uint32_t)g * NS * 2;
    const int64_t base = (b * L + t0) * (int64_t)G * NS + (int64_t)g * NS;
    const __amdgpu_buffer_rsrc_t rB = rsrc(B + base, bytes), rC = rsrc(C + base, bytes);
    {
      const int It = tile_i(ti), Jt = tile_j(ti);
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const u32x4 a = __builtin_amdgcn_raw_buffer_load_b128(rB, (int)((16 * Jt + li) * row + (32 * kb + 8 * lg) * 2), 0, 0);
        const u32x4 bb = __builtin_amdgcn_raw_buffer_load_b128(rC, (int)((16 * It + li) * row + (32 * kb + 8 * lg) * 2), 0, 0);
        acc = mfma(as_bf16x8(a), as_bf16x8(bb), acc);
      }
      *(f32x4*)(cb + (blk * kTiles + ti) * kTileFloats + 4 * l) = acc;
    }
  }
}

// ---------------------------------------------------------------- fp32 activations
//
// ssd_chunk_f32_kernel: the chunked restatement, work items, segments and state
// hand-offs of ssd_chunk_kernel (one head per workgroup), for fp32 activations on
// fp32 MFMA (v_mfma_f32_16x16x4_f32: fp32 products and sums, so the chunked form
// carries fp32 rounding only). Operand layouts:
//   A[16 x 4]: lane l holds A[l % 16][l / 16]; B[4 x 16]: lane l holds
//   B[l / 16][l % 16]; D[16 x 16]: lane l holds D[4 (l / 16) + r][l % 16].
// With one float per lane and operand, each phase picks its own assignment of
// the contraction index k to the lane groups lg (any works if A and B agree):
//   Y^T = S_in C^T: k = lg <-> state n = 16 nt + 4 lg + r, so the A operand is the
//     state accumulator value hacc[nt][r] itself, and the B operand for r = 0..3
//     is one 16-byte read of row i of C (sCf, row-major);
//   S^T = exp(cs_last) S^T + B^T (w x) and Y^T += X^T M^T: k = lg <-> token
//     j = 16 jb + 4 lg + kk (kk = 0..3): the B^T operand (sBt, B transposed at
//     staging) and the M operand (sMf, row-major) are 16-byte reads for kk = 0..3,
//     and x[j][p] for the 16 (jb, kk) is read once per chunk and serves both;
//     Y^T += X^T M^T takes only the blocks jb <= it (M is lower triangular).
// The state is kept as S^T tiles in the accumulators (rows n, columns p), which
// puts S[p = 16 wq + li][n = 16 nt + 4 lg + r] in lane l, register r of tile nt:
// the layout of ssd_chunk_kernel, so the state moves in and out alike.
// Per chunk: after barrier A (chunk staged), the x operands; the mask of the C B^T
// tiles into M; Y^T = S_in C^T; the state update; barrier B (M complete); the
// gate and D x from this chunk's z and x; Y^T += X^T M^T; y into LDS; the switch
// of item after an item's last chunk; barrier C (every wave has read x and z);
// the next chunk staged from its prefetch registers; barrier A.
// LDS: B^T, C, x, z, y and M of a chunk in fp32 (142 KB, one workgroup per
// compute unit); row pitches 8 dwords past a multiple of 64, where 16-byte reads
// of 16 rows at once are conflict-free, except B^T, whose 16-byte blocks are
// swizzled (bt_at) so that its transposing writes are conflict-free too.
constexpr int LBT = Q;       // row pitch (fp32) of sBt: B^T [state][token], 16-byte blocks swizzled
// sBt row n holds its 16 blocks of 4 tokens with block b at position b ^ bt_swz(n): the
// 16 lanes of a transposing staging write (rows 4 nb + e) and of an operand read (rows
// 16 nt + li) then all land on distinct banks (unswizzled, rows 4 apart at any pitch
// that keeps 16-byte alignment share banks: up to 16-way conflicts on the writes)
__device__ __forceinline__ int bt_swz(int n) { return ((n & 15) + (n >> 4)) & 15; }
__device__ __forceinline__ int bt_at(int n, int j) { return n * LBT + 4 * ((j >> 2) ^ bt_swz(n)); }
constexpr int LCF = NS + 8;  // row pitch of sCf: C [token][state]
constexpr int LXF = P + 8;   // row pitch of sXf, sZf, sYf: [token][head_dim]
constexpr int LMF = Q + 8;   // row pitch of sMf: M [token i][token j]

__device__ __forceinline__ f32x4 mfma_f32(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 ld_f32x4(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
}

// One chunk's staged global loads of one thread (coalesced: 32 lanes cover a
// 512-byte row of B or C, 16 lanes a 256-byte row of x or z).
struct PrefetchF {
  f32x4 b[2][4];     // B rows 32 it + 4 (tid / 32) + u, states 4 (tid % 32) .. + 3
  f32x4 c[8];        // C rows 8 it + tid / 32, states 4 (tid % 32) .. + 3
  f32x4 x[4], z[4];  // x / z rows 16 it + tid / 16, columns 4 (tid % 16) .. + 3
  f32x4 g[3];        // the C B^T tiles this wave masks
  float dt;
};

template <int MODE>
__global__ __launch_bounds__(256, 1) void ssd_chunk_f32_kernel(SsdKF k) {
  constexpr bool Y = MODE != kLocal;  // the pass computes y (kLocal: only the state)
  constexpr int NW = 4, NT = 3;
  __shared__ __attribute__((aligned(16))) float sBt[NS * LBT];
  __shared__ __attribute__((aligned(16))) float sCf[Q * LCF];
  __shared__ __attribute__((aligned(16))) float sXf[Q * LXF];
  __shared__ __attribute__((aligned(16))) float sZf[Q * LXF];
  __shared__ __attribute__((aligned(16))) float sYf[Q * LXF];
  __shared__ __attribute__((aligned(16))) float sMf[Q * LMF];
  __shared__ __attribute__((aligned(16))) float sCS[Q], sDT[Q], sW[Q], sE[Q];
  __shared__ int sTicket[3];

  const int tid = threadIdx.x, w = __builtin_amdgcn_readfirstlane(tid >> 6), wq = w, l = tid & 63, li = l & 15,
            lg = l >> 4;
  const int L = (int)k.L, H = (int)k.H, G = (int)k.G;
  const bool gate = k.z != nullptr;

  // the work queues, as in ssd_chunk_kernel
  auto qindex = [&]() { return __builtin_amdgcn_readfirstlane((int)(blockIdx.x % (unsigned)kargs_f()->nq)); };
  auto qcounter = [&]() { return kargs_f()->queue + (MODE == kLocal ? 256 : 0) + 16 * qindex(); };
  auto qfirst = [&]() {
    return __builtin_amdgcn_readfirstlane((int)((unsigned)(qindex() * kargs_f()->nchains) / (unsigned)kargs_f()->nq));
  };
  auto qchains = [&]() {
    const unsigned q = (unsigned)qindex(), n = (unsigned)kargs_f()->nchains, nq = (unsigned)kargs_f()->nq;
    return __builtin_amdgcn_readfirstlane((int)((q + 1) * n / nq - q * n / nq));
  };
  auto qitems = [&]() { return (MODE == kLocal ? kargs_f()->nseg - 1 : kargs_f()->nseg) * qchains(); };

  if (tid == 0) sTicket[0] = (int)atomicAdd(qcounter(), 1u);
  __syncthreads();
  int cur = __builtin_amdgcn_readfirstlane(sTicket[0]);
  if (cur >= qitems()) return;
  int nxt = -1;

  // row bytes and elements per batch row
  const int Hd = H >> k.hshift;  // dt_raw columns (the caller's heads)
  const uint32_t bc_row = (uint32_t)(G * NS * 4), xz_row = (uint32_t)(H * P * 4), dt_row = (uint32_t)(Hd * 4);
  const uint32_t bc_bat = (uint32_t)L * (G * NS), xz_bat = (uint32_t)L * (H * P), dt_bat = (uint32_t)L * Hd;
  const int nb = tid & 31, jq = tid >> 5;  // staging of B and C: 16-byte piece, row
  const int xp = tid & 15, xr = tid >> 4;  // staging of x, z and y: 16-byte piece, row

  int tb = 0, th = 0, tg = 0, tt = 0;  // target of the loads in flight (as in ssd_chunk_kernel)
  auto tgt_rsrc = [&](const float* base, uint32_t bat, uint32_t col, uint32_t rowb, bool on = true) {
    const int left = on ? L - tt : 0;
    return rsrc((const char*)(base + (uint64_t)tb * bat + col) + (uint32_t)tt * rowb,
                left > 0 ? (uint32_t)left * rowb - col * 4 : 0u);
  };
  auto load_b = [&](PrefetchF& pf) {
    const __amdgpu_buffer_rsrc_t rB = tgt_rsrc(k.B, bc_bat, (uint32_t)tg * NS, bc_row);
#pragma unroll
    for (int it = 0; it < 2; ++it)
#pragma unroll
      for (int u = 0; u < 4; ++u) pf.b[it][u] = ld_f32x4(rB, (uint32_t)(32 * it + 4 * jq + u) * bc_row + nb * 16);
  };
  auto load_c = [&](PrefetchF& pf) {
    const __amdgpu_buffer_rsrc_t rC = tgt_rsrc(k.C, bc_bat, (uint32_t)tg * NS, bc_row);
#pragma unroll
    for (int it = 0; it < 8; ++it) pf.c[it] = ld_f32x4(rC, (uint32_t)(8 * it + jq) * bc_row + nb * 16);
  };
  auto load_g = [&](PrefetchF& pf) {
    const float* blk =
        kargs_f()->cb + (((int64_t)tb * kargs_f()->nchunks + tt / Q) * G + tg) * (kTiles * kTileFloats);
    const __amdgpu_buffer_rsrc_t rG = rsrc(blk, tt < L ? kTiles * kTileFloats * 4 : 0u);
#pragma unroll
    for (int u = 0; u < NT; ++u) {
      const int ti = w + NW * u < kTiles ? w + NW * u : w;
      pf.g[u] = ld_f32x4(rG, (uint32_t)(ti * 64 + l) * 16);
    }
  };
  auto load_x = [&](PrefetchF& pf) {
    const __amdgpu_buffer_rsrc_t rX = tgt_rsrc(k.x, xz_bat, (uint32_t)th * P, xz_row);
    const __amdgpu_buffer_rsrc_t rD =
        tgt_rsrc(k.dt, dt_bat, (uint32_t)(th >> kargs_f()->hshift), dt_row, wq == kDecayWave);
#pragma unroll
    for (int it = 0; it < 4; ++it) pf.x[it] = ld_f32x4(rX, (uint32_t)(16 * it + xr) * xz_row + xp * 16);
    pf.dt = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rD, (int)(l * dt_row), 0, 0));
  };
  auto load_z = [&](PrefetchF& pf) {
    const __amdgpu_buffer_rsrc_t rZ = tgt_rsrc(gate ? k.z : k.x, xz_bat, (uint32_t)th * P, xz_row);
#pragma unroll
    for (int it = 0; it < 4; ++it) pf.z[it] = ld_f32x4(rZ, (uint32_t)(16 * it + xr) * xz_row + xp * 16);
  };
  __amdgpu_buffer_rsrc_t ry_prev = rsrc(k.y, 0);
  auto store_y = [&]() {
#pragma unroll
    for (int it = 0; it < 4; ++it)
      __builtin_amdgcn_raw_buffer_store_b128(*(const u32x4*)(sYf + (16 * it + xr) * LXF + 4 * xp), ry_prev,
                                             (int)((uint32_t)(16 * it + xr) * xz_row + xp * 16), 0, 2);
  };

  int b = 0, h = 0, g = 0, c = 0, c_end = 0, seg = 0;
  float A2 = 0.f, bias = 0.f, Dh = 0.f;
  auto set_item = [&](int it) {
    const KArgsF* kk = kargs_f();
    const int nch = qchains();
    seg = it / nch;
    const int ch = qfirst() + it % nch;
    b = ch / H;
    h = ch % H;
    g = h / kk->heads_per_group;
    c = seg * kk->seg_chunks;
    c_end = min(c + kk->seg_chunks, max((L + Q - 1) / Q, 1));
    const int hp = h >> kk->hshift;  // the caller's head
    A2 = -expf(kk->A_log[hp]) * kLog2e;
    bias = kk->dt_bias[hp];
    Dh = kk->D[hp];
  };

  // Chunk at token tt from the prefetch registers into LDS (B transposed); wave
  // kDecayWave adds the steps, their inclusive cumulative sum (exp2 domain), the
  // row scales exp(cs) and the state update's weights w_j = exp(cs_last - cs_j) dt_j.
  auto stage = [&](PrefetchF& pf) {
#pragma unroll
    for (int it = 0; it < 2; ++it)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        *(f32x4*)(sBt + bt_at(4 * nb + e, 32 * it + 4 * jq)) =
            f32x4{pf.b[it][0][e], pf.b[it][1][e], pf.b[it][2][e], pf.b[it][3][e]};
    if constexpr (Y) {
#pragma unroll
      for (int it = 0; it < 8; ++it) *(f32x4*)(sCf + (8 * it + jq) * LCF + 4 * nb) = pf.c[it];
    }
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      *(f32x4*)(sXf + (16 * it + xr) * LXF + 4 * xp) = pf.x[it];
      if constexpr (Y) *(f32x4*)(sZf + (16 * it + xr) * LXF + 4 * xp) = pf.z[it];
    }
    if (wq == kDecayWave) {
      const int nt_valid = max(0, min(Q, L - tt));
      const float dtv = l < nt_valid ? softplus(pf.dt + bias) : 0.0f;
      const float cs = wave_inclusive_sum(dtv * A2);
      const float cs_last = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(cs), 63));
      sDT[l] = dtv;
      sCS[l] = cs;
      sE[l] = fast_exp2(cs);
      sW[l] = fast_exp2(cs_last - cs) * dtv;
    }
  };

  f32x4 hacc[8];
  const int64_t s_lane = (int64_t)(16 * wq + li) * NS + 4 * lg;
  // the entering and leaving state, as in ssd_chunk_kernel (chain_state_in / _out: the
  // same flags, give-up word and carry; a chain is one head)
  float lam = 0.0f;  // kLocal: the item's decay sum so far (exp2 domain)
  auto state_in = [&]() {
    chain_state_in<MODE>(hacc, tid, seg, (int64_t)b * H + h, (int64_t)b * H + h, s_lane, sTicket[2]);
    lam = 0.0f;
  };
  auto state_out = [&]() {
    chain_state_out<MODE>(hacc, tid, seg, (int64_t)b * H + h, (int64_t)b * H + h, s_lane, lam);
  };

  set_item(cur);
  tb = b; th = h; tg = g; tt = c * Q;
  PrefetchF pf;
  load_b(pf);
  if constexpr (Y) {
    load_c(pf);
    load_g(pf);
  }
  load_x(pf);
  if constexpr (Y) load_z(pf);
  stage(pf);
  state_in();
  if (tid == 0) sTicket[1] = (int)atomicAdd(qcounter(), 1u);
  __syncthreads();
  {
    const int t = __builtin_amdgcn_readfirstlane(sTicket[1]);
    nxt = t < qitems() ? t : -1;
  }

  for (;;) {
    const int t0 = c * Q;
    const bool last = c + 1 == c_end;
    // ---- after barrier A: chunk c is in LDS; loads go to the next chunk
    int ticket = 0;
    if (!last) {
      tt = t0 + Q;
    } else if (nxt >= 0) {
      const int qn = qchains(), ns = nxt / qn, nch = qfirst() + nxt % qn;
      tb = nch / H;
      th = nch % H;
      tg = th / kargs_f()->heads_per_group;
      tt = ns * kargs_f()->seg_chunks * Q;
      if (tid == 0) ticket = (int)atomicAdd(qcounter(), 1u);
    } else {
      tt = L;
    }
    if constexpr (Y) store_y();
    load_b(pf);
    if constexpr (Y) load_z(pf);

    // x[j = 16 jb + 4 lg + kk][p = 16 wq + li]: operand of the state update and of X^T M^T
    float xv[4][4];
#pragma unroll
    for (int jb = 0; jb < 4; ++jb)
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) xv[jb][kk] = sXf[(16 * jb + 4 * lg + kk) * LXF + 16 * wq + li];

    // ---- G tiles -> M[i][j] = G[i][j] exp(cs_i - cs_j) dt_j (j <= i), fp32, row-major;
    // wave w takes tiles w, w + 4, w + 8 (a wave with two masks its first again)
#pragma unroll
    for (int u = 0; u < (Y ? NT : 0); ++u) {
      const int ti = w + NW * u < kTiles ? w + NW * u : w;
      const int It = tile_i(ti), Jt = tile_j(ti);
      const int i = 16 * It + li;
      const float csi = sCS[i];
      const f32x4 csj = *(const f32x4*)(sCS + 16 * Jt + 4 * lg);
      const f32x4 dtj = *(const f32x4*)(sDT + 16 * Jt + 4 * lg);
      f32x4 m;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int j = 16 * Jt + 4 * lg + r;
        const float v = pf.g[u][r] * fast_exp2(fminf(csi - csj[r], 0.0f)) * dtj[r];
        m[r] = j <= i ? v : 0.0f;
      }
      *(f32x4*)(sMf + i * LMF + 16 * Jt + 4 * lg) = m;
    }

    if constexpr (Y) {
      load_c(pf);
      load_g(pf);
    }
    float ei[4];
#pragma unroll
    for (int it = 0; it < 4; ++it) ei[it] = sE[16 * it + li];
    f32x4 wv[4];
#pragma unroll
    for (int jb = 0; jb < 4; ++jb) wv[jb] = *(const f32x4*)(sW + 16 * jb + 4 * lg);
    const float dec_last = sE[Q - 1];
    if constexpr (!Y) lam += sCS[Q - 1];

    // ---- Y^T = S_in C^T, columns scaled by exp(cs_i); per state tile the four rows of
    // C are read first, then the 16 MFMAs go to the four output tiles in turn
    f32x4 yacc[4];
#pragma unroll
    for (int it = 0; it < 4; ++it) yacc[it] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int nt = 0; nt < (Y ? 8 : 0); ++nt) {
      f32x4 cv[4];
#pragma unroll
      for (int it = 0; it < 4; ++it) cv[it] = *(const f32x4*)(sCf + (16 * it + li) * LCF + 16 * nt + 4 * lg);
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int it = 0; it < 4; ++it) yacc[it] = mfma_f32(hacc[nt][r], cv[it][r], yacc[it]);
    }
#pragma unroll
    for (int it = 0; it < 4; ++it) {
#pragma unroll
      for (int r = 0; r < 4; ++r) yacc[it][r] *= ei[it];
    }

    load_x(pf);
    // ---- S^T = exp(cs_last) S^T + B^T (w x)
    float wx[4][4];
#pragma unroll
    for (int jb = 0; jb < 4; ++jb)
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) wx[jb][kk] = wv[jb][kk] * xv[jb][kk];
    // (two state tiles at a time: two accumulator chains)
#pragma unroll
    for (int nt = 0; nt < 8; nt += 2) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        hacc[nt][r] *= dec_last;
        hacc[nt + 1][r] *= dec_last;
      }
#pragma unroll
      for (int jb = 0; jb < 4; ++jb) {
        const f32x4 b0 = *(const f32x4*)(sBt + bt_at(16 * nt + li, 16 * jb + 4 * lg));
        const f32x4 b1 = *(const f32x4*)(sBt + bt_at(16 * nt + 16 + li, 16 * jb + 4 * lg));
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          hacc[nt] = mfma_f32(b0[kk], wx[jb][kk], hacc[nt]);
          hacc[nt + 1] = mfma_f32(b1[kk], wx[jb][kk], hacc[nt + 1]);
        }
      }
    }

    __syncthreads();  // ---- barrier B: M complete; no wave reads sBt, sCf or the decays again

    // the epilogue's gate and D x, which do not depend on Y^T and so can run beside the
    // MFMAs below: y = (Y + D x) silu(z) = Y g + D x g. x and z are read here, not held
    // through the MFMA phases; barrier C keeps the next chunk's staging behind these
    // reads. (Staging before X^T M^T, beside its MFMAs, measured 2.5% slower.)
    f32x4 gv[4], dxg[4];
#pragma unroll
    for (int it = 0; it < (Y ? 4 : 0); ++it) {
      const f32x4 xe = *(const f32x4*)(sXf + (16 * it + li) * LXF + 16 * wq + 4 * lg);
      const f32x4 ze = *(const f32x4*)(sZf + (16 * it + li) * LXF + 16 * wq + 4 * lg);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        gv[it][r] = gate ? silu(ze[r]) : 1.0f;
        dxg[it][r] = Dh * xe[r] * gv[it][r];
      }
    }
    // ---- Y^T += X^T M^T over the blocks jb <= it
#pragma unroll
    for (int it = 0; it < (Y ? 4 : 0); ++it) {
#pragma unroll
      for (int jb = 0; jb < 4; ++jb) {
        if (jb > it) continue;
        const f32x4 mv = *(const f32x4*)(sMf + (16 * it + li) * LMF + 16 * jb + 4 * lg);
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) yacc[it] = mfma_f32(xv[jb][kk], mv[kk], yacc[it]);
      }
    }
    // ---- epilogue: lane holds y[i = 16 it + li][16 wq + 4 lg + r]
    if constexpr (Y) {
      const __amdgpu_buffer_rsrc_t rY = rsrc((const char*)(k.y + (uint64_t)b * xz_bat + h * P) + (uint32_t)t0 * xz_row,
                                             (uint32_t)(L - t0) * xz_row - h * P * 4);
#pragma unroll
      for (int it = 0; it < 4; ++it) {
        f32x4 v;
#pragma unroll
        for (int r = 0; r < 4; ++r) v[r] = fmaf(yacc[it][r], gv[it][r], dxg[it][r]);
        *(f32x4*)(sYf + (16 * it + li) * LXF + 16 * wq + 4 * lg) = v;
      }
      ry_prev = rY;
    }
    const bool finished = last && nxt < 0;
    if (last) {
      state_out();
      if (!finished) {
        if (tid == 0) sTicket[1] = ticket;
        set_item(nxt);
        state_in();
        __syncthreads();
        const int t = __builtin_amdgcn_readfirstlane(sTicket[1]);
        nxt = t < qitems() ? t : -1;
      }
    } else {
      ++c;
    }
    __syncthreads();  // ---- barrier C: every wave has read this chunk's x and z
    stage(pf);
    __syncthreads();  // ---- barrier A of the next chunk
    if (finished) break;
  }
  if constexpr (Y) store_y();
}

// ssd_cb_kernel for fp32 B and C on fp32 MFMA, in the same tile layout:
//   cb[blk][ti][l][r] = sum_n C[t0 + 16 It + l % 16][n] B[t0 + 16 Jt + 4 (l / 16) + r][n],
// computed as the transposed tile (A operand from rows of B, B operand from rows
// of C; k = lane group <-> n = 16 nb + 4 lg + kk). Also clears the work queues.
__global__ __launch_bounds__(640) void ssd_cb_f32_kernel(const float* __restrict__ B, const float* __restrict__ C,
                                                         float* __restrict__ cb, int L, int G, int nchunks, int64_t nblk,
                                                         unsigned* __restrict__ q, int nq, unsigned give_up) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < nq; i += gridDim.x * blockDim.x)
    q[i] = i == 128 ? give_up : 0u;
  const int ti = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)), l = threadIdx.x & 63, li = l & 15,
            lg = l >> 4;
  const uint32_t row = (uint32_t)(G * NS * 4);
  for (int64_t blk = blockIdx.x; blk < nblk; blk += gridDim.x) {
    const int g = (int)(blk % G), c = (int)((blk / G) % nchunks);
    const int64_t b = blk / ((int64_t)G * nchunks);
    const int t0 = c * Q;
    const uint32_t bytes = (uint32_t)(L - t0) * row - (uint32_t)g * NS * 4;
    const int64_t base = (b * L + t0) * (int64_t)G * NS + (int64_t)g * NS;
    const __amdgpu_buffer_rsrc_t rB = rsrc(B + base, bytes), rC = rsrc(C + base, bytes);
    const int It = tile_i(ti), Jt = tile_j(ti);
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) {
      const f32x4 a = ld_f32x4(rB, (uint32_t)(16 * Jt + li) * row + (16 * nb + 4 * lg) * 4);
      const f32x4 cc = ld_f32x4(rC, (uint32_t)(16 * It + li) * row + (16 * nb + 4 * lg) * 4);
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) acc = mfma_f32(a[kk], cc[kk], acc);
    }
    *(f32x4*)(cb + (blk * kTiles + ti) * kTileFloats + 4 * l) = acc;
  }
}

// state_dim 64..127 on the chunk kernels: rows of nin entries (B, C, the entering
// state) copied into rows of NS with zeros after them, and the leaving state's rows
// cut back to nout entries. With B, C and the entering state zero in states
// nin..NS-1, those state columns stay exactly zero (each update scales zero and adds
// a zero product) and add exact zeros to every C.B^T and C.S sum, so states 0..nin-1
// and y are the unpadded problem's. One workgroup of NS threads per row.
template <typename T>
__global__ __launch_bounds__(NS) void pad_state_rows_kernel(const T* __restrict__ src, T* __restrict__ dst,
                                                            int64_t rows, int nin) {
  const int j = threadIdx.x;
  for (int64_t r = blockIdx.x; r < rows; r += gridDim.x) dst[r * NS + j] = j < nin ? src[r * nin + j] : T(0);
}

__global__ __launch_bounds__(NS) void unpad_state_rows_kernel(const float* __restrict__ src, float* __restrict__ dst,
                                                              int64_t rows, int nout) {
  const int j = threadIdx.x;
  if (j >= nout) return;
  for (int64_t r = blockIdx.x; r < rows; r += gridDim.x) dst[r * nout + j] = src[r * NS + j];
}

namespace {

// log2(head_dim / 64): a head of 64 * 2^k columns is 2^k heads of 64 columns that
// share its step, decay and D (its columns are independent given those); -1 for
// any other head_dim
int head_shift(int64_t P_) {
  for (int k = 0; k < 16; ++k)
    if (P_ == (int64_t)P << k) return k;
  return -1;
}

// The problem seen as heads of P = 64 columns (x, y and the states keep their layout)
SSDArgs by_64_columns(const SSDArgs& a) {
  SSDArgs v = a;
  v.H = a.H << head_shift(a.P);
  v.P = P;
  return v;
}

// How the chains are cut into segments and how many workgroups take them. A
// chain (one head of one batch row) is sequential; with fewer chains than
// compute units some units idle whatever is done, and with a few more (say 1.25
// per unit) whole chains leave some units with two and the rest idle half the
// time. Cutting every chain into segments that any workgroup may take evens
// the load: the cost model counts rounds of items over one workgroup per unit,
// plus one chunk of overhead per item.
//
// Few chains (fewer than units, say one batch row of 80 heads) leave units idle in
// one pass, since a chain's segments wait for each other. Then two passes can win:
// the first computes every segment but the last from a zero state, only its state
// update (the kLocal kernel, about kLocalCost of a chunk's time per chunk), and
// the second runs all segments at once, each from its entering state folded from
// the first pass's (kFolded). The model counts the rounds of each pass.
struct SsdPlan {
  int hpw, nchains, seg_chunks, nseg, nq, grid;
  bool split;      // bf16: the precise form (state and w x as two bf16 parts each)
  bool two_pass;   // kLocal and kFolded passes (else one kChained pass)
  int grid_local;  // workgroups of the kLocal pass
  size_t queue_bytes, carry_bytes, lam_bytes, cb_bytes, ws_bytes;
  size_t cb_off, pad_off;                // workspace offsets of the C B^T tiles and the padded copies
  size_t pad_bc_bytes, pad_state_bytes;  // state_dim < NS: each padded B, C and state copy
};

// per-chunk time of the kLocal pass relative to a full chunk, in percent (bf16, fp32;
// measured at one batch row of the Mamba-2 2.7B layer: 0.57 and 0.42)
constexpr int64_t kLocalCostBf16 = 55, kLocalCostF32 = 45;

// (a: the problem in heads of 64 columns; allow_two: two passes may be chosen)
SsdPlan ssd_plan(const SSDArgs& a, bool allow_two = true) {
  const bool f32 = !a.bf16;
  int dev = 0, ncu = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || ncu <= 0)
    ncu = 256;
  SsdPlan p{};
  // One head per workgroup. Two (a chain is then a pair of neighbouring heads of one
  // batch row that share a group of B and C) on request: measured at the Mamba-2 2.7B
  // layer they are 5-10% slower, the second wave per SIMD adding LDS waits rather
  // than hiding latency.
  const int64_t hpg = a.H / a.G;
  // (fp32 activations: one head per workgroup, the only form of that kernel)
  // The precise form on request (bf16; one head per workgroup).
  p.split = !f32 && knob(kKnobSsdSplitState) != 0;
  p.hpw = (!f32 && !p.split && knob(kKnobSsdHeadsPerWorkgroup) == 2 && a.H % 2 == 0 && hpg % 2 == 0) ? 2 : 1;
  const int64_t nchains = a.batch * a.H / p.hpw, nchunks = std::max<int64_t>((a.L + Q - 1) / Q, 1);
  p.nchains = (int)nchains;
  // Two workgroups per unit (the occupancy the one-head kernel is built for) with
  // many chains; the two-head kernel and the fp32 kernel fill a unit's LDS with one.
  int64_t grid = (!f32 && p.hpw == 1 && nchains >= 2 * (int64_t)ncu) ? 2 * ncu : ncu;
  int64_t best_seg = nchunks, best_ns = 1, best_cost = 0;
  auto queues = [&](int64_t g) { return std::max<int64_t>(1, std::min<int64_t>({8, nchains, g})); };
  {
    // rounds of items in the fullest queue over its workgroups (with many more chains
    // than workgroups, whole chains win: cutting them only adds hand-offs)
    const int64_t nq = queues(grid), qch = (nchains + nq - 1) / nq, qwg = std::max<int64_t>(grid / nq, 1);
    auto cost = [&](int64_t sc, int64_t ns) {
      const int64_t rounds = (ns * qch + qwg - 1) / qwg;
      return std::max(rounds * (sc + 1), nchunks + ns);
    };
    int64_t best = cost(nchunks, 1);
    for (int64_t s = 2; s <= std::min<int64_t>(nchunks, 64) && s * nchains < (int64_t(1) << 30); ++s) {
      const int64_t sc = (nchunks + s - 1) / s, ns = (nchunks + sc - 1) / sc;
      const int64_t cst = cost(sc, ns);
      if (cst * 100 < best * 97) {  // a cut must win by 3% to be taken
        best = cst;
        best_seg = sc;
        best_ns = ns;
      }
    }
    best_cost = best;
  }
  // Two passes (one head per workgroup): rounds of the first pass's items (every
  // segment but the last) at kLocalCost per chunk, then of the second's; in hundredths
  // of a chunk. bf16 may also run two workgroups per unit (the kernel is built for
  // that occupancy): a pass whose items fit one per unit costs one round as before;
  // otherwise each round of up to two items per unit costs 1.5 rounds (two
  // workgroups sharing a unit each run at about two thirds of the speed: measured
  // 1.49-1.55 at one and two batch rows of the Mamba-2 2.7B layer).
  bool two_pass = false;
  int64_t seg2 = nchunks, ns2 = 1, grid2 = ncu;
  const int tp = allow_two ? knob(kKnobSsdTwoPass) : 1;  // 1: one pass; 2: two passes
  if (p.hpw == 1 && tp != 1) {
    const int64_t lc = f32 ? kLocalCostF32 : kLocalCostBf16;
    int64_t best2 = -1;
    for (int per_cu = 1; per_cu <= (f32 ? 1 : 2); ++per_cu) {
      const int64_t g2 = per_cu * (int64_t)ncu, nq = queues(g2), qch = (nchains + nq - 1) / nq;
      const int64_t cu_q = std::max<int64_t>(ncu / nq, 1);  // units per queue
      auto pass = [&](int64_t items, int64_t chunk_cost) {
        if (items <= cu_q) return items > 0 ? chunk_cost : int64_t(0);
        const int64_t slots = per_cu * cu_q, rounds = (items + slots - 1) / slots;
        return per_cu == 1 ? rounds * chunk_cost : rounds * chunk_cost * 3 / 2;
      };
      for (int64_t s = 1; s <= std::min<int64_t>(nchunks, 64) && s * nchains < (int64_t(1) << 30); ++s) {
        const int64_t sc = (nchunks + s - 1) / s, ns = (nchunks + sc - 1) / sc;
        // the fold between the passes: a launch (about 1.3 chunks) and, per chain and
        // segment, a state read and written (64 KB: 0.007 of a chunk at 4 TB/s)
        const int64_t fold = ns > 1 ? 130 + (ns - 1) * nchains * 71 / 100 : 0;
        const int64_t cst = pass((ns - 1) * qch, lc * sc + 100) + fold + pass(ns * qch, 100 * sc + 100);
        if (best2 < 0 || cst < best2) {
          best2 = cst;
          seg2 = sc;
          ns2 = ns;
          grid2 = g2;
        }
      }
    }
    // (the one-pass cost, best_cost, in whole chunks; two passes must win by 3%)
    two_pass = tp == 2 || (ns2 > 1 && best2 * 100 < best_cost * 100 * 97);
  }
  if (two_pass) {
    best_seg = seg2;
    best_ns = ns2;
    grid = grid2;
  }
  // tuning overrides: chunks per segment, workgroups
  if (const int64_t sc = knob(kKnobSsdSegmentChunks); sc > 0) {
    best_seg = std::min(sc, nchunks);
    best_ns = (nchunks + best_seg - 1) / best_seg;
    if (best_ns * nchains >= (int64_t(1) << 30)) best_seg = nchunks, best_ns = 1;
  }
  if (const int64_t wg = knob(kKnobSsdWorkgroups); wg > 0) grid = std::min<int64_t>(wg, 1 << 20);
  p.two_pass = two_pass;
  p.seg_chunks = (int)best_seg;
  p.nseg = (int)best_ns;
  p.nq = (int)queues(grid);
  // no more workgroups than the fullest queue has items, per queue
  const int64_t qch = (nchains + p.nq - 1) / p.nq;
  p.grid = (int)std::min<int64_t>(grid, (int64_t)p.nq * best_ns * qch);
  p.grid_local = (int)std::max<int64_t>(1, std::min<int64_t>(grid, (int64_t)p.nq * (best_ns - 1) * qch));
  // queue words: 8 counters (16 apart), the give-up word at 128, then a flag per
  // chain from 256 (one pass) or the first pass's 8 counters there (two passes)
  p.queue_bytes = ((size_t)(256 + std::max(p.nchains, 128)) * 4 + 255) / 256 * 256;
  const size_t state_bytes = (size_t)(a.batch * a.H) * P * NS * 4;
  p.carry_bytes = p.nseg > 1 ? (two_pass ? (size_t)(p.nseg - 1) : 1) * state_bytes : 0;
  p.lam_bytes = two_pass && p.nseg > 1 ? ((size_t)(p.nseg - 1) * (size_t)(a.batch * a.H) * 4 + 255) / 256 * 256 : 0;
  p.cb_bytes = (size_t)a.batch * (size_t)((a.L + Q - 1) / Q) * (size_t)a.G * kTiles * kTileFloats * 4;
  p.cb_off = p.queue_bytes + p.carry_bytes + p.lam_bytes;
  p.pad_off = p.cb_off + p.cb_bytes;
  // state_dim below NS: B and C padded to NS states, and the entering and leaving
  // states as [batch, H, P, NS] (after the C B^T tiles, 256-byte aligned)
  const size_t es = f32 ? 4 : 2;
  p.pad_bc_bytes = a.N < NS ? ((size_t)(a.batch * a.L * a.G) * NS * es + 255) / 256 * 256 : 0;
  p.pad_state_bytes = a.N < NS ? state_bytes : 0;
  p.ws_bytes = p.pad_off + 2 * p.pad_bc_bytes + 2 * p.pad_state_bytes;
  // a capped workspace (the allocation-free entry point's scratch) that two passes
  // would overflow: one pass, which needs less
  if (two_pass && a.ws_cap && p.ws_bytes > a.ws_cap) return ssd_plan(a, false);
  return p;
}

}  // namespace

bool ssd_chunk_supported(const SSDArgs& a) {
  // buffer offsets are 32-bit: each batch row of x / z / y / B / C must stay below 2^31 bytes.
  // A sequence of length 0 goes to the token loop, which only passes the state through:
  // the chunk kernels size their resources as (L - t0) rows less the head's or group's
  // column offset, which needs at least one token row.
  // head_dim 64 * 2^k: each head is 2^k heads of 64 columns (by_64_columns).
  const int64_t es = a.bf16 ? 2 : 4;
  const int hsh = head_shift(a.P);
  const int64_t row_x = a.L * a.H * a.P * es, row_bc = a.L * a.G * NS * es;
  // state_dim 64..NS: below NS, zero-padded in the workspace (pad_state_rows_kernel).
  return (a.bf16 || knob(kKnobSsdF32TokenLoop) == 0) && a.L > 0 && hsh >= 0 && a.N >= 64 && a.N <= NS &&
         a.states == nullptr && a.H <= (1 << 24) && (a.batch * a.H << hsh) <= (1 << 24) &&
         row_x < (int64_t(1) << 31) && row_bc < (int64_t(1) << 31);
}

size_t ssd_chunk_ws(const SSDArgs& a) { return a.batch == 0 ? 0 : ssd_plan(by_64_columns(a)).ws_bytes; }

// The kernel arguments both chunk kernels share: workspace layout, sizes, plan.
template <typename K>
void fill_common(K& k, const SSDArgs& a, const SsdPlan& p, int hshift, void* ws) {
  k.queue = (unsigned*)ws;
  k.carry = p.nseg > 1 ? (float*)((char*)ws + p.queue_bytes) : nullptr;
  k.lam = p.lam_bytes ? (float*)((char*)ws + p.queue_bytes + p.carry_bytes) : nullptr;
  k.cb = (float*)((char*)ws + p.cb_off);
  k.L = a.L; k.H = a.H; k.G = a.G; k.heads_per_group = (int)(a.H / a.G);
  k.nchunks = (int)((a.L + Q - 1) / Q);
  k.nchains = p.nchains; k.seg_chunks = p.seg_chunks; k.nseg = p.nseg; k.nq = p.nq;
  k.hshift = hshift;
  k.nstates = (int)(a.batch * a.H);
}

// Between the two passes: the segments' entering states (ssd_fold_states_kernel)
template <typename K>
void launch_fold(const K& k, hipStream_t s) {
  const int64_t threads = (int64_t)k.nstates * (P * NS / 4);
  hipLaunchKernelGGL(ssd_fold_states_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s, k.carry, k.lam,
                     k.h0, k.nstates, k.nseg - 1);
}

// fp32 activations: ssd_cb_f32_kernel and ssd_chunk_f32_kernel on the same plan
// (a: the problem in heads of 64 columns; hshift: log2 of the caller's head_dim / 64)
hipError_t launch_ssd_chunk_f32(const SSDArgs& a, const SsdPlan& p, int hshift, void* ws, hipStream_t s) {
  SsdKF k{};
  k.x = (const float*)a.x; k.dt = (const float*)a.dt; k.dt_bias = a.dt_bias; k.A_log = a.A_log;
  k.B = (const float*)a.B; k.C = (const float*)a.C; k.D = a.D; k.z = (const float*)a.z;
  k.h0 = a.h0; k.y = (float*)a.y; k.h_out = a.h_out;
  fill_common(k, a, p, hshift, ws);
  const int64_t nblk = a.batch * (int64_t)k.nchunks * a.G;
  hipLaunchKernelGGL(ssd_cb_f32_kernel, dim3((unsigned)std::max<int64_t>(1, std::min<int64_t>(nblk, 1 << 20))),
                     dim3(640), 0, s, (const float*)a.B, (const float*)a.C, (float*)k.cb, (int)a.L, (int)a.G, k.nchunks, nblk,
                     k.queue, (int)(p.queue_bytes / 4), knob(kKnobSsdGiveUp) != 0 ? 1u : 0u);
  if (!p.two_pass) {
    hipLaunchKernelGGL(ssd_chunk_f32_kernel<kChained>, dim3((unsigned)p.grid), dim3(256), 0, s, k);
  } else {
    if (p.nseg > 1) {
      hipLaunchKernelGGL(ssd_chunk_f32_kernel<kLocal>, dim3((unsigned)p.grid_local), dim3(256), 0, s, k);
      launch_fold(k, s);
    }
    hipLaunchKernelGGL(ssd_chunk_f32_kernel<kFolded>, dim3((unsigned)p.grid), dim3(256), 0, s, k);
  }
  return hipGetLastError();
}

// bf16 activations: ssd_cb_kernel and ssd_chunk_kernel (a, hshift as for the fp32 launch)
static hipError_t launch_ssd_chunk_bf16(const SSDArgs& a, const SsdPlan& p, int hshift, void* ws, hipStream_t s) {
  SsdK k{};
  k.x = (const uint16_t*)a.x; k.dt = (const uint16_t*)a.dt; k.dt_bias = a.dt_bias; k.A_log = a.A_log;
  k.B = (const uint16_t*)a.B; k.C = (const uint16_t*)a.C; k.D = a.D; k.z = (const uint16_t*)a.z;
  k.h0 = a.h0; k.y = (uint16_t*)a.y; k.h_out = a.h_out;
  fill_common(k, a, p, hshift, ws);
  const int64_t nblk = a.batch * (int64_t)k.nchunks * a.G;
  // (at least one workgroup: it also clears the queues)
  hipLaunchKernelGGL(ssd_cb_kernel, dim3((unsigned)std::max<int64_t>(1, std::min<int64_t>(nblk, 1 << 20))), dim3(640),
                     0, s, (const uint16_t*)a.B, (const uint16_t*)a.C, (float*)k.cb, (int)a.L, (int)a.G, k.nchunks, nblk,
                     k.queue, (int)(p.queue_bytes / 4), knob(kKnobSsdGiveUp) != 0 ? 1u : 0u);
  if (p.split) {
    if (p.two_pass) {
      if (p.nseg > 1) {
        hipLaunchKernelGGL((ssd_chunk_kernel<1, kLocal, true>), dim3((unsigned)p.grid_local), dim3(256), kCkBytes, s,
                           k);
        launch_fold(k, s);
      }
      hipLaunchKernelGGL((ssd_chunk_kernel<1, kFolded, true>), dim3((unsigned)p.grid), dim3(256), kCkBytes, s, k);
    } else {
      hipLaunchKernelGGL((ssd_chunk_kernel<1, kChained, true>), dim3((unsigned)p.grid), dim3(256), kCkBytes, s, k);
    }
  } else if (p.two_pass) {
    if (p.nseg > 1) {
      hipLaunchKernelGGL((ssd_chunk_kernel<1, kLocal>), dim3((unsigned)p.grid_local), dim3(256), kCkBytes, s, k);
      launch_fold(k, s);
    }
    hipLaunchKernelGGL((ssd_chunk_kernel<1, kFolded>), dim3((unsigned)p.grid), dim3(256), kCkBytes, s, k);
  } else if (p.hpw == 2) {
    hipLaunchKernelGGL((ssd_chunk_kernel<2, kChained>), dim3((unsigned)p.grid), dim3(512), kCkBytes, s, k);
  } else {
    hipLaunchKernelGGL((ssd_chunk_kernel<1, kChained>), dim3((unsigned)p.grid), dim3(256), kCkBytes, s, k);
  }
  return hipGetLastError();
}

static hipError_t launch_ssd_chunk_padded(const SSDArgs& a, const SsdPlan& p, int hshift, void* ws, hipStream_t s);

hipError_t launch_ssd_chunk(const SSDArgs& a_caller, void* ws, hipStream_t s) {
  if (a_caller.batch == 0) return hipSuccess;
  const SSDArgs a = by_64_columns(a_caller);
  const int hshift = head_shift(a_caller.P);
  const SsdPlan p = ssd_plan(a);
  if (a.N < NS) return launch_ssd_chunk_padded(a, p, hshift, ws, s);
  return a.bf16 ? launch_ssd_chunk_bf16(a, p, hshift, ws, s) : launch_ssd_chunk_f32(a, p, hshift, ws, s);
}

// state_dim below NS: B, C and the entering state padded with zero states into the
// workspace (after the C B^T tiles), the chunk kernels run at NS on those copies,
// and the leaving state's first N entries per row go to the caller.
static hipError_t launch_ssd_chunk_padded(const SSDArgs& a, const SsdPlan& p, int hshift, void* ws, hipStream_t s) {
  char* base = (char*)ws + p.pad_off;
  void* pB = base;
  void* pC = base + p.pad_bc_bytes;
  float* pH0 = (float*)(base + 2 * p.pad_bc_bytes);
  float* pHo = (float*)(base + 2 * p.pad_bc_bytes + p.pad_state_bytes);
  const int64_t bc_rows = a.batch * a.L * a.G, st_rows = a.batch * a.H * P;
  auto grid = [](int64_t rows) { return dim3((unsigned)std::max<int64_t>(1, std::min<int64_t>(rows, 1 << 16))); };
  if (a.bf16) {
    hipLaunchKernelGGL(pad_state_rows_kernel<uint16_t>, grid(bc_rows), dim3(NS), 0, s, (const uint16_t*)a.B,
                       (uint16_t*)pB, bc_rows, (int)a.N);
    hipLaunchKernelGGL(pad_state_rows_kernel<uint16_t>, grid(bc_rows), dim3(NS), 0, s, (const uint16_t*)a.C,
                       (uint16_t*)pC, bc_rows, (int)a.N);
  } else {
    hipLaunchKernelGGL(pad_state_rows_kernel<float>, grid(bc_rows), dim3(NS), 0, s, (const float*)a.B, (float*)pB,
                       bc_rows, (int)a.N);
    hipLaunchKernelGGL(pad_state_rows_kernel<float>, grid(bc_rows), dim3(NS), 0, s, (const float*)a.C, (float*)pC,
                       bc_rows, (int)a.N);
  }
  if (a.h0)
    hipLaunchKernelGGL(pad_state_rows_kernel<float>, grid(st_rows), dim3(NS), 0, s, a.h0, pH0, st_rows, (int)a.N);
  SSDArgs v = a;
  v.N = NS;
  v.B = pB;
  v.C = pC;
  v.h0 = a.h0 ? pH0 : nullptr;
  v.h_out = pHo;
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  e = v.bf16 ? launch_ssd_chunk_bf16(v, p, hshift, ws, s) : launch_ssd_chunk_f32(v, p, hshift, ws, s);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(unpad_state_rows_kernel, grid(st_rows), dim3(NS), 0, s, pHo, a.h_out, st_rows, (int)a.N);
  return hipGetLastError();
}

}  // namespace sscan
