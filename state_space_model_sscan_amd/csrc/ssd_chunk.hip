// ssd_chunk.hip -- the Mamba-2 SSD prompt scan on MFMA for gfx950 (bf16 in, fp32 state).
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
// Per chunk, between two barriers:
//   after barrier A (chunk staged in LDS: B, C and x row-major, C once more in the
//   k order of the S C^T operand, cumulative decay):
//     - x^T fragments and the epilogue's x values move from LDS to registers;
//     - G^T = B C^T on MFMA (10 lower-triangular 16x16 tiles over the 4 waves),
//       masked and scaled into M[i, j] = G[i, j] exp(cs_i - cs_j) dt_j (bf16, LDS);
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
#include <stdlib.h>
#include <string.h>

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
constexpr int LDC = NS + 16;  // row pitch of sC and sCk: 72 dwords, where 16-byte reads of
                              // 16 rows (the MFMA operands) are conflict-free
constexpr int LDX = P + 8;   // row pitch of sX
constexpr int LDM = Q + 8;   // row pitch of sM
constexpr size_t kCkBytes = (size_t)Q * LDC * 2;
// The wave that computes the chunk's steps and decays while staging: one of the
// two waves whose third G tile is a repeat (waves 0 and 1 have three tiles).
constexpr int kDecayWave = 3;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));

struct SsdK {
  const uint16_t* x;
  const uint16_t* dt;
  const float* dt_bias;
  const float* A_log;
  const uint16_t* B;
  const uint16_t* C;
  const float* D;
  const uint16_t* z;
  const float* h0;
  uint16_t* y;
  float* h_out;
  unsigned* queue;  // [16 q]: next item of queue q; [128]: a wait gave up; [256 + ch]: segments of chain ch done
  float* carry;     // [chains, P, NS]: the state a segment hands to the next one
  int64_t L, H, G;
  int heads_per_group;
  int nchains;      // batch * H
  int seg_chunks;   // chunks per segment
  int nseg;         // segments per chain
  int nq;           // work queues; workgroup i serves queue i % nq, which holds chains
                    // [q nchains / nq, (q + 1) nchains / nq): item i of a queue with n chains is
                    // segment i / n of its chain i % n
};

// Position of token t of a chunk in k order (see the note on the transposing load):
// within each group of 8, token 8g + t sits at 8g + (t even ? t/2 : 4 + t/2).
__device__ __forceinline__ int kslot(int t) { return (t & ~7) | ((t & 1) << 2) | ((t & 7) >> 1); }

typedef __attribute__((address_space(4))) const SsdK KArgs;
// The kernel's arguments, read again from the argument segment: used where a
// value is needed rarely, so that it does not hold a scalar register.
__device__ __forceinline__ KArgs* kargs() {
  uint64_t v = (uint64_t)__builtin_amdgcn_kernarg_segment_ptr();
  asm volatile("" : "+s"(v));
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v), hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (KArgs*)(((uint64_t)hi << 32) | lo);
}

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

// One chunk's staged global loads of one thread, in flight during the previous
// chunk. Coalesced: 16 lanes cover a 256-byte row of B or C (an instruction, 4
// rows), 8 lanes a 128-byte row of x (8 rows), so each load touches a few cache
// lines rather than one per lane. B, C: rows 16w + 4it + l/16, piece l%16; x and
// z: rows 16w + 8it + l/8, piece l%8; dt (wave kDecayWave only): token l.
struct Prefetch {
  u32x4 b[4], c[4], x[2], z[2];
  uint32_t dt;  // raw bf16 bits
};

}  // namespace

__global__ __launch_bounds__(256, 2) void ssd_chunk_kernel(SsdK k) {
  __shared__ __attribute__((aligned(16))) uint16_t sB[Q * LDB];
  __shared__ __attribute__((aligned(16))) uint16_t sC[Q * LDC];
  // C again, each row in the k order of the Y^T = S C^T operand: positions
  // 32kb + 8lg + e hold states 32kb + 4lg + e (e < 4) and 32kb + 16 + 4lg + e - 4
  // (e >= 4), so that operand is one 16-byte read (the state accumulators fix
  // that order)
  // (dynamic LDS of kCkBytes: its size then does not lower the occupancy the code
  // is compiled for, which schedules this kernel better)
  extern __shared__ __attribute__((aligned(16))) uint16_t sCk[];
  __shared__ __attribute__((aligned(16))) uint16_t sX[Q * LDX];
  __shared__ __attribute__((aligned(16))) uint16_t sM[Q * LDM];
  __shared__ __attribute__((aligned(16))) uint16_t sZ[Q * LDX];  // z of the chunk
  __shared__ __attribute__((aligned(16))) uint16_t sY[Q * LDX];  // y of the chunk, stored after the next barrier
  __shared__ __attribute__((aligned(16))) float sCS[Q], sDT[Q], sW[Q], sE[Q];
  __shared__ int sTicket[2];  // [0]: the first item; [1]: the item after the current one

  // the wave index through readfirstlane: a scalar, so branches on it stay uniform
  const int tid = threadIdx.x, w = __builtin_amdgcn_readfirstlane(tid >> 6), l = tid & 63, li = l & 15,
            lg = l >> 4;
  // 32-bit sizes: the host guarantees each batch row of every tensor is < 2^31 bytes
  const int L = (int)k.L, H = (int)k.H, G = (int)k.G;
  const bool gate = k.z != nullptr;

  // This workgroup's queue (the dispatcher deals workgroups to the eight compute
  // dies in turn, so the queues match the dies and a die's L2 serves neighbouring
  // heads, which share B and C): its counter, first chain, chains and items.
  // Computed where needed from the argument segment, so that none holds a
  // scalar register through the chunk loop.
  // (32-bit: chains < 2^24 and queues <= 8; readfirstlane marks the quotients
  // uniform, so buffer resources built from them stay scalar)
  auto qindex = [&]() { return __builtin_amdgcn_readfirstlane((int)(blockIdx.x % (unsigned)kargs()->nq)); };
  auto qcounter = [&]() { return kargs()->queue + 16 * qindex(); };
  auto qfirst = [&]() {
    return __builtin_amdgcn_readfirstlane((int)((unsigned)(qindex() * kargs()->nchains) / (unsigned)kargs()->nq));
  };
  auto qchains = [&]() {
    const unsigned q = (unsigned)qindex(), n = (unsigned)kargs()->nchains, nq = (unsigned)kargs()->nq;
    return __builtin_amdgcn_readfirstlane((int)((q + 1) * n / nq - q * n / nq));
  };
  auto qitems = [&]() { return kargs()->nseg * qchains(); };

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

  const uint32_t bc_row = (uint32_t)(G * NS * 2), xz_row = (uint32_t)(H * P * 2), dt_row = (uint32_t)(H * 2);
  // elements per batch row
  const uint32_t bc_bat = (uint32_t)L * (G * NS), xz_bat = (uint32_t)L * (H * P), dt_bat = (uint32_t)L * H;
  const int bc_r = 16 * w + (l >> 4), bc_p = l & 15;  // staging row (+ 4 it) and piece of B, C
  const int x_r = 16 * w + (l >> 3), x_p = l & 7;     // staging row (+ 8 it) and piece of x
  const uint32_t bc_lane = (uint32_t)(bc_r * bc_row + bc_p * 16);
  const uint32_t x_lane = (uint32_t)(x_r * xz_row + x_p * 16);
  const uint32_t dt_lane = (uint32_t)(l * dt_row);

  // Global access goes through buffer resources based at a chunk's first token
  // row and this chain's first column, ending at the sequence end (the host
  // guarantees each batch row is < 2^31 bytes): rows past the end read zeros
  // and drop their stores in hardware, and the lane offsets stay uniform.
  // Target of the loads in flight: chain (tb, th, tg), first token tt (tt >= L:
  // none; every load reads zeros).
  int tb = 0, th = 0, tg = 0, tt = 0;
  auto tgt_rsrc = [&](const uint16_t* base, uint32_t bat, uint32_t col, uint32_t rowb, bool on = true) {
    const int left = on ? L - tt : 0;
    return rsrc((const char*)(base + (uint64_t)tb * bat + col) + (uint32_t)tt * rowb,
                left > 0 ? (uint32_t)left * rowb - col * 2 : 0u);
  };
  auto load_b = [&](Prefetch& pf) {
    const __amdgpu_buffer_rsrc_t rB = tgt_rsrc(k.B, bc_bat, (uint32_t)tg * NS, bc_row);
#pragma unroll
    for (int it = 0; it < 4; ++it)
      pf.b[it] = __builtin_amdgcn_raw_buffer_load_b128(rB, (int)(bc_lane + it * 4 * bc_row), 0, 0);
  };
  auto load_c = [&](Prefetch& pf) {
    const __amdgpu_buffer_rsrc_t rC = tgt_rsrc(k.C, bc_bat, (uint32_t)tg * NS, bc_row);
#pragma unroll
    for (int it = 0; it < 4; ++it)
      pf.c[it] = __builtin_amdgcn_raw_buffer_load_b128(rC, (int)(bc_lane + it * 4 * bc_row), 0, 0);
  };
  auto load_x = [&](Prefetch& pf) {
    const __amdgpu_buffer_rsrc_t rX = tgt_rsrc(k.x, xz_bat, (uint32_t)th * P, xz_row);
    // only the decay wave uses dt: the other waves' resource is empty (no memory access)
    const __amdgpu_buffer_rsrc_t rD = tgt_rsrc(k.dt, dt_bat, (uint32_t)th, dt_row, w == kDecayWave);
#pragma unroll
    for (int it = 0; it < 2; ++it)
      pf.x[it] = __builtin_amdgcn_raw_buffer_load_b128(rX, (int)(x_lane + it * 8 * xz_row), 0, 0);
    pf.dt = __builtin_amdgcn_raw_buffer_load_b16(rD, (int)dt_lane, 0, 0);
  };
  // z of the target chunk, staged like x (without a gate: loads of x, unused)
  auto load_z = [&](Prefetch& pf) {
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
      __builtin_amdgcn_raw_buffer_store_b128(lds128(sY + (x_r + 8 * it) * LDX + x_p * 8), ry_prev,
                                             (int)(x_lane + it * 8 * xz_row), 0, 2);
  };

  // The current item: chain (b, h) of group g, chunks [c, c_end); per-head constants.
  int b = 0, h = 0, g = 0, c = 0, c_end = 0;
  int seg = 0;
  float A2 = 0.f, bias = 0.f, Dh = 0.f;
  auto set_item = [&](int it) {
    const KArgs* kk = kargs();
    const int nch = qchains();
    seg = it / nch;
    const int ch = qfirst() + it % nch;
    b = ch / H;
    h = ch % H;
    g = h / kk->heads_per_group;
    c = seg * kk->seg_chunks;
    c_end = min(c + kk->seg_chunks, max((L + Q - 1) / Q, 1));  // seqlen 0: one empty chunk
    A2 = -expf(kk->A_log[h]) * kLog2e;  // decay per unit step, exp2 domain
    bias = kk->dt_bias[h];
    Dh = kk->D[h];
  };

  // Chunk at token tt from the prefetch registers into LDS; wave kDecayWave adds the
  // steps, their inclusive cumulative sum (exp2 domain) and the derived decays.
  auto stage = [&](Prefetch& pf) {
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      *(u32x4*)(sB + (bc_r + 4 * it) * LDB + bc_p * 8) = pf.b[it];
      *(u32x4*)(sC + (bc_r + 4 * it) * LDC + bc_p * 8) = pf.c[it];
      // states 8 bc_p + e: piece q = bc_p % 4 of the 32 states 32kb.. (kb = bc_p / 4)
      // goes to positions 32kb + 16 (q % 2) + 4 (q / 2) and 8 further on
      const int pk = 32 * (bc_p >> 2) + 16 * (bc_p & 1) + 4 * ((bc_p >> 1) & 1);
      *(u32x2*)(sCk + (bc_r + 4 * it) * LDC + pk) = u32x2{pf.c[it][0], pf.c[it][1]};
      *(u32x2*)(sCk + (bc_r + 4 * it) * LDC + pk + 8) = u32x2{pf.c[it][2], pf.c[it][3]};
    }
#pragma unroll
    for (int it = 0; it < 2; ++it) {
      *(u32x4*)(sX + (x_r + 8 * it) * LDX + x_p * 8) = pf.x[it];
      *(u32x4*)(sZ + (x_r + 8 * it) * LDX + x_p * 8) = pf.z[it];
    }
    if (w == kDecayWave) {
      const int nt_valid = max(0, min(Q, L - tt));
      const float dtv = l < nt_valid ? softplus(lo_f(pf.dt) + bias) : 0.0f;  // past the end: a zero step
      const float cs = wave_inclusive_sum(dtv * A2);
      const float cs_last = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(cs), 63));
      sDT[l] = dtv;
      sCS[l] = cs;
      sE[l] = fast_exp2(cs);
      sW[kslot(l)] = fast_exp2(cs_last - cs) * dtv;  // in k order
    }
  };

  // state slice: hacc[nt][r] = S[p = 16w + li][n = 16nt + 4lg + r]; stored as [chain, p, n]
  f32x4 hacc[8];
  const int64_t s_lane = (int64_t)(16 * w + li) * NS + 4 * lg;
  // The entering state of the current item: the caller's (or zeros) for a first
  // segment, else the one the previous segment left in carry, once its flag says
  // so. The producer of that segment holds an item dequeued earlier than this
  // one, so it is running and never waits on this workgroup: the wait ends. Its
  // bound (2^20 polls, about a second) only guarantees that the kernel
  // terminates; a wait that gives up raises queue[128], which ends every other.
  // carry and the flags move through device-coherent loads and stores (the sc1
  // cache policy, as device-scope atomics use), which need no cache write-back
  // or invalidation (either would flush the L2 that the other workgroups share);
  // carry moves in 16-byte pieces, so the write-through goes out in whole
  // 64-byte segments.
  auto state_in = [&]() {
    const int64_t ch = (int64_t)b * H + h;
    if (seg > 0) {
      if (tid == 0) {
        unsigned* flag = kargs()->queue + 256 + ch;
        bool done = false;
        for (int n = 0; n < (1 << 20) && !done; ++n) {
          done = __hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= (unsigned)seg ||
                 __hip_atomic_load(kargs()->queue + 128, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0u;
          if (!done) __builtin_amdgcn_s_sleep(2);
        }
        if (!done) __hip_atomic_store(kargs()->queue + 128, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      __syncthreads();
      const __amdgpu_buffer_rsrc_t rS = rsrc(kargs()->carry + ch * (P * NS), P * NS * 4);
#pragma unroll
      for (int nt = 0; nt < 8; ++nt)
        hacc[nt] = __builtin_bit_cast(
            f32x4, __builtin_amdgcn_raw_buffer_load_b128(rS, (int)((s_lane + 16 * nt) * 4), 0, kDeviceCoherent));
    } else if (kargs()->h0) {
      const float* src = kargs()->h0 + ch * (P * NS) + s_lane;
#pragma unroll
      for (int nt = 0; nt < 8; ++nt) hacc[nt] = *(const f32x4*)(src + 16 * nt);
    } else {
#pragma unroll
      for (int nt = 0; nt < 8; ++nt) hacc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    // The loads complete here: otherwise every chunk would wait for them (and
    // for the chunk loads queued behind them) before it first reads the state.
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) asm volatile("" : "+v"(hacc[nt]));
  };
  // The leaving state: to the caller after the last segment, else to carry and
  // then the flag. Every thread waits until its stores are complete (visible to
  // the device) before the barrier; thread 0 raises the flag after it.
  auto state_out = [&]() {
    const int64_t ch = (int64_t)b * H + h;
    if (seg + 1 < kargs()->nseg) {
      const __amdgpu_buffer_rsrc_t rS = rsrc(kargs()->carry + ch * (P * NS), P * NS * 4);
#pragma unroll
      for (int nt = 0; nt < 8; ++nt)
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, hacc[nt]), rS, (int)((s_lane + 16 * nt) * 4), 0,
                                               kDeviceCoherent);
      __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the stores above have completed
      __syncthreads();
      if (tid == 0) __hip_atomic_store(kargs()->queue + 256 + ch, (unsigned)(seg + 1), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    } else {
      float* dst = kargs()->h_out + ch * (P * NS) + s_lane;
#pragma unroll
      for (int nt = 0; nt < 8; ++nt) *(f32x4*)(dst + 16 * nt) = hacc[nt];
    }
  };

  // the tiles of M above the diagonal block row stay zero
  for (int e = tid; e < Q * LDM; e += 256) sM[e] = 0;

  set_item(cur);
  tb = b; th = h; tg = g; tt = c * Q;
  Prefetch pf;
  load_b(pf);
  load_c(pf);
  load_x(pf);
  load_z(pf);
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
      tb = nch / H;
      th = nch % H;
      tg = th / kargs()->heads_per_group;
      tt = ns * kargs()->seg_chunks * Q;
      if (tid == 0) ticket = (int)atomicAdd(qcounter(), 1u);  // the item after that
    } else {
      tt = L;
    }
    store_y();  // the previous chunk's y (sY complete since barrier A)
    load_b(pf);
    load_z(pf);

    // x^T fragments (A operand of Y^T += X^T M^T; k = j = 32kb + 8lg + kperm(e)) by
    // two transposing loads each, and the epilogue's x values (8 bytes of row 16it + li)
    u32x4 xa[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int k0 = 32 * kb + 8 * lg;
      const u32x2 lo = lds_tr(sX + (k0 + 2 * (li >> 2)) * LDX + 16 * w + 4 * (li & 3));
      const u32x2 hi = lds_tr(sX + (k0 + 1 + 2 * (li >> 2)) * LDX + 16 * w + 4 * (li & 3));
      xa[kb] = u32x4{lo[0], lo[1], hi[0], hi[1]};
    }
    u32x2 xe[4], zkeep[4];
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      xe[it] = lds64(sX + (16 * it + li) * LDX + 16 * w + 4 * lg);
      zkeep[it] = lds64(sZ + (16 * it + li) * LDX + 16 * w + 4 * lg);
    }

    // ---- G^T tiles -> M (lower triangle): wave w takes tiles w, w+4, w+8. Waves 2
    // and 3 have no tile w+8 and compute tile w twice, writing the same values
    // again: a branch around the third tile would split the phase into pieces
    // that each wait for all of their LDS reads.
    {
      f32x4 acc[3];
      int Jt[3], It[3];
#pragma unroll
      for (int u = 0; u < 3; ++u) {
        const int ti = w + 4 * u < 10 ? w + 4 * u : w;
        // ti -> (Jt, It), It >= Jt: (0,0) (0,1) (0,2) (0,3) (1,1) (1,2) (1,3) (2,2) (2,3) (3,3)
        Jt[u] = ti < 4 ? 0 : (ti < 7 ? 1 : (ti < 9 ? 2 : 3));
        It[u] = ti < 4 ? ti : (ti < 7 ? ti - 3 : (ti < 9 ? ti - 5 : 3));
        acc[u] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
      // the mask's cumulative sums and steps, read before the MFMAs so that their
      // latency hides behind them (the scheduler would otherwise sink the reads to
      // their use)
      float csi[3];
      f32x4 csj[3], dtj[3];
#pragma unroll
      for (int u = 0; u < 3; ++u) {
        csi[u] = sCS[16 * It[u] + li];
        csj[u] = *(const f32x4*)(sCS + 16 * Jt[u] + 4 * lg);
        dtj[u] = *(const f32x4*)(sDT + 16 * Jt[u] + 4 * lg);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int u = 0; u < 3; ++u) {
          const bf16x8 a = as_bf16x8(lds128(sB + (16 * Jt[u] + li) * LDB + 32 * kb + 8 * lg));
          const bf16x8 bb = as_bf16x8(lds128(sC + (16 * It[u] + li) * LDC + 32 * kb + 8 * lg));
          acc[u] = mfma(a, bb, acc[u]);
        }
#pragma unroll
      for (int u = 0; u < 3; ++u) {
        // acc[r] = G[i][j], i = 16It + li, j = 16Jt + 4lg + r
        const int i = 16 * It[u] + li;
        float m[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int j = 16 * Jt[u] + 4 * lg + r;
          // computed for every lane and selected (the clamp keeps masked entries finite)
          const float v = acc[u][r] * fast_exp2(fminf(csi[u] - csj[u][r], 0.0f)) * dtj[u][r];
          m[r] = j <= i ? v : 0.0f;
        }
        // columns in k order: j = 16Jt + 4lg + r sits at 16Jt + 8(lg/2) + kslot(4(lg%2) + r)
        uint16_t* row = sM + i * LDM + 16 * Jt[u] + 8 * (lg >> 1) + 2 * (lg & 1);
        *(uint32_t*)row = pack2(m[0], m[2]);
        *(uint32_t*)(row + 4) = pack2(m[1], m[3]);
      }
    }

    load_c(pf);
    // ---- Y^T = S_in C^T, columns scaled by exp(cs_i). A operand: the state,
    // k = n in {32kb + 4lg + r} U {32kb + 16 + 4lg + r} (the accumulator layout);
    // B operand: C[i][n] for the same n, 16 bytes of row i of sCk.
    // the row scales and the state update's weights, read before the MFMAs
    float ei[4];
#pragma unroll
    for (int it = 0; it < 4; ++it) ei[it] = sE[16 * it + li];
    f32x4 wj[2][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      wj[kb][0] = *(const f32x4*)(sW + 32 * kb + 8 * lg);
      wj[kb][1] = *(const f32x4*)(sW + 32 * kb + 8 * lg + 4);
    }
    const float dec_last = sE[Q - 1];
    __builtin_amdgcn_sched_barrier(0);
    f32x4 yacc[4];
#pragma unroll
    for (int it = 0; it < 4; ++it) yacc[it] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      u32x4 sv;
      sv[0] = pack2(hacc[2 * kb][0], hacc[2 * kb][1]);
      sv[1] = pack2(hacc[2 * kb][2], hacc[2 * kb][3]);
      sv[2] = pack2(hacc[2 * kb + 1][0], hacc[2 * kb + 1][1]);
      sv[3] = pack2(hacc[2 * kb + 1][2], hacc[2 * kb + 1][3]);
      const bf16x8 aop = as_bf16x8(sv);
#pragma unroll
      for (int it = 0; it < 4; ++it) {
        yacc[it] = mfma(aop, as_bf16x8(lds128(sCk + (16 * it + li) * LDC + 32 * kb + 8 * lg)), yacc[it]);
      }
    }
#pragma unroll
    for (int it = 0; it < 4; ++it) {
#pragma unroll
      for (int r = 0; r < 4; ++r) yacc[it][r] *= ei[it];
    }

    load_x(pf);
    // ---- S = exp(cs_last) S + B^T (w x). A operand: B^T rows n = 16nt + li, k = j
    // (transposing loads of B); B operand: w_j x[j][16w + li] from the x^T fragments
    // (both in k order; sW holds w in k order).
    bf16x8 wxb[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const f32x4 w0 = wj[kb][0], w1 = wj[kb][1];
      const u32x4 v = xa[kb];
      wxb[kb] = as_bf16x8(u32x4{pack2(lo_f(v[0]) * w0[0], hi_f(v[0]) * w0[1]),
                                pack2(lo_f(v[1]) * w0[2], hi_f(v[1]) * w0[3]),
                                pack2(lo_f(v[2]) * w1[0], hi_f(v[2]) * w1[1]),
                                pack2(lo_f(v[3]) * w1[2], hi_f(v[3]) * w1[3])});
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
        hacc[nt] = mfma(as_bf16x8(u32x4{lo[0], lo[1], hi[0], hi[1]}), wxb[kb], hacc[nt]);
      }
    }

    __syncthreads();  // ---- barrier B: M complete; no wave reads sB, sC, sX or the decays again

    // ---- Y^T += X^T M^T (M[i][j] = 0 for j > i: skip the upper blocks)
#pragma unroll
    for (int it = 0; it < 4; ++it) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        if (kb == 1 && it < 2) continue;
        const bf16x8 mb = as_bf16x8(lds128(sM + (16 * it + li) * LDM + 32 * kb + 8 * lg));
        yacc[it] = mfma(as_bf16x8(xa[kb]), mb, yacc[it]);
      }
    }
    // ---- epilogue: lane holds y[i = 16it + li][16w + 4lg + r]; y = (Y + D x) silu(z)
    {
      const __amdgpu_buffer_rsrc_t rY = rsrc((const char*)(k.y + (uint64_t)b * xz_bat + h * P) + (uint32_t)t0 * xz_row,
                                             (uint32_t)(L - t0) * xz_row - h * P * 2);
#pragma unroll
      for (int it = 0; it < 4; ++it) {
        const float xs[4] = {lo_f(xe[it][0]), hi_f(xe[it][0]), lo_f(xe[it][1]), hi_f(xe[it][1])};
        const float zs[4] = {lo_f(zkeep[it][0]), hi_f(zkeep[it][0]), lo_f(zkeep[it][1]), hi_f(zkeep[it][1])};
        float v[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) v[r] = fmaf(Dh, xs[r], yacc[it][r]) * (gate ? silu(zs[r]) : 1.0f);
        *(u32x2*)(sY + (16 * it + li) * LDX + 16 * w + 4 * lg) = u32x2{pack2(v[0], v[1]), pack2(v[2], v[3])};
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
  store_y();  // the last chunk's y
}

// Zeroes the queue counters, the give-up word and the per-chain flags (a kernel, not a memset, so
// that the call can be captured in a graph).
__global__ void ssd_queue_reset(unsigned* q, int n) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) q[i] = 0;
}

namespace {

// How the chains are cut into segments and how many workgroups take them. A
// chain (one head of one batch row) is sequential; with fewer chains than
// compute units some units idle whatever is done, and with a few more (say 1.25
// per unit) whole chains leave some units with two and the rest idle half the
// time. Cutting every chain into segments that any workgroup may take evens
// the load: the cost model counts rounds of items over one workgroup per unit,
// plus one chunk of overhead per item.
struct SsdPlan {
  int nchains, seg_chunks, nseg, nq, grid;
  size_t queue_bytes, ws_bytes;
};

SsdPlan ssd_plan(const SSDArgs& a) {
  int dev = 0, ncu = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || ncu <= 0)
    ncu = 256;
  SsdPlan p{};
  const int64_t nchains = a.batch * a.H, nchunks = std::max<int64_t>((a.L + Q - 1) / Q, 1);
  p.nchains = (int)nchains;
  int64_t grid = nchains < 2 * (int64_t)ncu ? ncu : 2 * ncu;  // two per unit (the occupancy the
                                                               // kernel is built for) with many chains
  int64_t best_seg = nchunks, best_ns = 1;
  auto queues = [&](int64_t g) { return std::max<int64_t>(1, std::min<int64_t>({8, nchains, g})); };
  if (nchains < 2 * (int64_t)ncu) {
    // rounds of items in the fullest queue over its workgroups
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
  }
  // tuning override "chunks per segment[,workgroups]"
  if (const char* e = getenv("SSCAN_SSD_SEGMENT")) {
    const int64_t sc = atoll(e);
    const char* comma = strchr(e, ',');
    if (sc > 0) {
      best_seg = std::min(sc, nchunks);
      best_ns = (nchunks + best_seg - 1) / best_seg;
      if (best_ns * nchains >= (int64_t(1) << 30)) best_seg = nchunks, best_ns = 1;
    }
    if (comma && atoll(comma + 1) > 0) grid = std::min<int64_t>(atoll(comma + 1), 1 << 20);
  }
  p.seg_chunks = (int)best_seg;
  p.nseg = (int)best_ns;
  p.nq = (int)queues(grid);
  // no more workgroups than the fullest queue has items, per queue
  const int64_t qitems = best_ns * ((nchains + p.nq - 1) / p.nq);
  p.grid = (int)std::min<int64_t>(grid, (int64_t)p.nq * qitems);
  p.queue_bytes = ((size_t)(256 + p.nchains) * 4 + 255) / 256 * 256;
  p.ws_bytes = p.queue_bytes + (p.nseg > 1 ? (size_t)p.nchains * P * NS * 4 : 0);
  return p;
}

}  // namespace

bool ssd_chunk_supported(const SSDArgs& a) {
  // buffer offsets are 32-bit: each batch row of x / z / y / B / C must stay below 2^31 bytes
  const int64_t row_x = a.L * a.H * P * 2, row_bc = a.L * a.G * NS * 2;
  return a.bf16 && a.P == P && a.N == NS && a.states == nullptr && a.batch * a.H <= (1 << 24) &&
         row_x < (int64_t(1) << 31) && row_bc < (int64_t(1) << 31);
}

size_t ssd_chunk_ws(const SSDArgs& a) { return a.batch == 0 ? 0 : ssd_plan(a).ws_bytes; }

hipError_t launch_ssd_chunk(const SSDArgs& a, void* ws, hipStream_t s) {
  if (a.batch == 0) return hipSuccess;
  const SsdPlan p = ssd_plan(a);
  SsdK k{};
  k.x = (const uint16_t*)a.x; k.dt = (const uint16_t*)a.dt; k.dt_bias = a.dt_bias; k.A_log = a.A_log;
  k.B = (const uint16_t*)a.B; k.C = (const uint16_t*)a.C; k.D = a.D; k.z = (const uint16_t*)a.z;
  k.h0 = a.h0; k.y = (uint16_t*)a.y; k.h_out = a.h_out;
  k.queue = (unsigned*)ws;
  k.carry = p.nseg > 1 ? (float*)((char*)ws + p.queue_bytes) : nullptr;
  k.L = a.L; k.H = a.H; k.G = a.G; k.heads_per_group = (int)(a.H / a.G);
  k.nchains = p.nchains; k.seg_chunks = p.seg_chunks; k.nseg = p.nseg; k.nq = p.nq;
  const int nwords = 256 + p.nchains;
  hipLaunchKernelGGL(ssd_queue_reset, dim3((unsigned)std::min(64, (nwords + 255) / 256)), dim3(256), 0, s, k.queue,
                     nwords);
  hipLaunchKernelGGL(ssd_chunk_kernel, dim3((unsigned)p.grid), dim3(256), kCkBytes, s, k);
  return hipGetLastError();
}

}  // namespace sscan
