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
// Mapping: one workgroup of 4 waves per (batch, head), walking the chunks in
// order. Wave w owns head_dim columns [16w, 16w+16): its slice of the state
// lives in fp32 MFMA accumulators (8 tiles of 16x16, state_dim 128) for the
// whole sequence. The output is computed transposed, Y^T = X^T M^T + S C^T, so
// that each lane ends up holding 4 neighbouring head_dim columns of one token
// row and stores them straight from registers.
//
// Per chunk, between two barriers:
//   after barrier A (chunk staged in LDS: B, C and x row-major, cumulative decay):
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
// Transposing LDS load (verified on gfx950): within each 16-lane group, if
// lane a supplies the address of 4 consecutive bf16 at row k0 + a/4, column
// c0 + 4(a%4) of a row-major tile, lane i receives rows k0..k0+3 of column c0 + i.
#include "device_common.hpp"
#include "launch.hpp"

namespace sscan {

namespace {

constexpr int Q = 64;        // tokens per chunk
constexpr int P = 64;        // head_dim
constexpr int NS = 128;      // state_dim
constexpr int LDB = NS + 24;  // row pitch (bf16) of sB, sC: 76 dwords = 12 mod 64, so
                              // 16 consecutive rows (MFMA operand reads) and the 4-row
                              // windows of the transposing loads both hit distinct banks
constexpr int LDX = P + 8;   // row pitch of sX
constexpr int LDM = Q + 8;   // row pitch of sM

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
  int64_t L, H, G;
  int heads_per_group;
  int nblocks;  // batch * H
};

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
// chunk. B, C: 4 pieces of 8 bf16 (row tid & 63, pieces (tid >> 6) + 4*it); x: 2
// pieces; dt: token tid & 63.
struct Prefetch {
  u32x4 b[4], c[4], x[2];
  uint32_t dt;  // raw bf16 bits
};

}  // namespace

__global__ __launch_bounds__(256, 2) void ssd_chunk_kernel(SsdK k) {
  __shared__ __attribute__((aligned(16))) uint16_t sB[Q * LDB];
  __shared__ __attribute__((aligned(16))) uint16_t sC[Q * LDB];
  __shared__ __attribute__((aligned(16))) uint16_t sX[Q * LDX];
  __shared__ __attribute__((aligned(16))) uint16_t sM[Q * LDM];
  __shared__ __attribute__((aligned(16))) float sCS[Q], sDT[Q], sW[Q], sE[Q];

  // block -> (batch, head): consecutive heads of one batch row share an XCD (and its L2)
  int lin = blockIdx.x;
  if (k.nblocks % 8 == 0) lin = (blockIdx.x % 8) * (k.nblocks / 8) + blockIdx.x / 8;
  const int64_t b = lin / k.H, h = lin % k.H;
  const int64_t g = h / k.heads_per_group;
  // the wave index through readfirstlane: a scalar, so branches on it stay uniform
  const int tid = threadIdx.x, w = __builtin_amdgcn_readfirstlane(tid >> 6), l = tid & 63, li = l & 15,
            lg = l >> 4;
  const int64_t L = k.L, H = k.H, G = k.G;
  const float A2 = -expf(k.A_log[h]) * kLog2e;  // decay per unit step, exp2 domain
  const float bias = k.dt_bias[h];
  const float Dh = k.D[h];
  const bool gate = k.z != nullptr;

  // Global access: buffer resources based at the chunk's first token row and
  // ending at the sequence end (the host guarantees each batch row is < 2^31 bytes).
  const uint16_t* Bb = k.B + b * L * G * NS;
  const uint16_t* Cb = k.C + b * L * G * NS;
  const uint16_t* Xb = k.x + b * L * H * P;
  const uint16_t* Zb = gate ? k.z + b * L * H * P : Xb;  // no gate: loads of x, unused
  uint16_t* Yb = k.y + b * L * H * P;
  const uint16_t* Db = k.dt + b * L * H;
  const uint32_t bc_row = (uint32_t)(G * NS * 2), xz_row = (uint32_t)(H * P * 2), dt_row = (uint32_t)(H * 2);
  auto chunk_rsrc = [&](const void* base, int64_t t0, uint32_t rowb) {
    const int64_t left = L - t0;
    return rsrc((const char*)base + t0 * rowb, left > 0 ? (uint64_t)left * rowb : 0);
  };
  const int row = l;   // staging row of this thread
  const int pc0 = w;   // its first 8-element piece; pieces pc0 + 4*it
  const uint32_t bc_lane = (uint32_t)(row * bc_row + (g * NS + pc0 * 8) * 2);
  const uint32_t x_lane = (uint32_t)(row * xz_row + (h * P + pc0 * 8) * 2);
  // epilogue layout: row 16*it + li, columns 16w + 4lg .. +3
  const uint32_t e_lane = (uint32_t)(li * xz_row + (h * P + 16 * w + 4 * lg) * 2);
  const uint32_t dt_lane = (uint32_t)(l * dt_row + h * 2);

  // The loads of chunk c, in four parts that the loop spreads over the phases of
  // the chunk before it, so that the address units never take them in one burst.
  auto load_b = [&](Prefetch& pf, int64_t c) {
    const __amdgpu_buffer_rsrc_t rB = chunk_rsrc(Bb, c * Q, bc_row);
#pragma unroll
    for (int it = 0; it < 4; ++it)
      pf.b[it] = __builtin_amdgcn_raw_buffer_load_b128(rB, (int)(bc_lane + it * 64), 0, 0);
  };
  auto load_c = [&](Prefetch& pf, int64_t c) {
    const __amdgpu_buffer_rsrc_t rC = chunk_rsrc(Cb, c * Q, bc_row);
#pragma unroll
    for (int it = 0; it < 4; ++it)
      pf.c[it] = __builtin_amdgcn_raw_buffer_load_b128(rC, (int)(bc_lane + it * 64), 0, 0);
  };
  auto load_x = [&](Prefetch& pf, int64_t c) {
    const __amdgpu_buffer_rsrc_t rX = chunk_rsrc(Xb, c * Q, xz_row), rD = chunk_rsrc(Db, c * Q, dt_row);
#pragma unroll
    for (int it = 0; it < 2; ++it)
      pf.x[it] = __builtin_amdgcn_raw_buffer_load_b128(rX, (int)(x_lane + it * 64), 0, 0);
    pf.dt = __builtin_amdgcn_raw_buffer_load_b16(rD, (int)dt_lane, 0, 0);
  };
  // z of chunk c in the epilogue's layout (4 bf16 of row 16*it + li)
  u32x2 zkeep[4];
  auto load_z = [&](u32x2 (&zz)[4], int64_t c) {
    const __amdgpu_buffer_rsrc_t rZ = chunk_rsrc(Zb, c * Q, xz_row);
#pragma unroll
    for (int it = 0; it < 4; ++it)
      zz[it] = __builtin_amdgcn_raw_buffer_load_b64(rZ, (int)(e_lane + it * 16 * xz_row), 0, 0);
  };

  // Chunk c from the prefetch registers into LDS; wave 0 adds the steps, their
  // inclusive cumulative sum (exp2 domain) and the derived decays.
  auto stage = [&](Prefetch& pf, int64_t c) {
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int pc = pc0 + 4 * it;
      *(u32x4*)(sB + row * LDB + pc * 8) = pf.b[it];
      *(u32x4*)(sC + row * LDB + pc * 8) = pf.c[it];
    }
#pragma unroll
    for (int it = 0; it < 2; ++it) *(u32x4*)(sX + row * LDX + (pc0 + 4 * it) * 8) = pf.x[it];
    if (w == 0) {
      const int nt_valid = (int)min((int64_t)Q, L - c * Q);
      const float dtv = l < nt_valid ? softplus(lo_f(pf.dt) + bias) : 0.0f;  // past the end: a zero step
      const float cs = wave_inclusive_sum(dtv * A2);
      const float cs_last = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(cs), 63));
      sDT[l] = dtv;
      sCS[l] = cs;
      sE[l] = fast_exp2(cs);
      sW[l] = fast_exp2(cs_last - cs) * dtv;
    }
  };

  // state slice: hacc[nt][r] = S[p = 16w + li][n = 16nt + 4lg + r]
  f32x4 hacc[8];
  if (k.h0) {
#pragma unroll
    for (int nt = 0; nt < 8; ++nt)
      hacc[nt] = *(const f32x4*)(k.h0 + ((b * H + h) * P + 16 * w + li) * NS + 16 * nt + 4 * lg);
  } else {
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) hacc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  // the tiles of M above the diagonal block row stay zero
  for (int e = tid; e < Q * LDM; e += 256) sM[e] = 0;

  const int64_t nchunks = (L + Q - 1) / Q;
  Prefetch pf;
  load_b(pf, 0);
  load_c(pf, 0);
  load_x(pf, 0);
  load_z(zkeep, 0);
  stage(pf, 0);
  __syncthreads();

  for (int64_t c = 0; c < nchunks; ++c) {
    const int64_t t0 = c * Q;
    // ---- after barrier A: chunk c is in LDS; the next chunk's B is requested
    load_b(pf, c + 1);

    // x^T fragments (A operand of Y^T += X^T M^T; k = j = 32kb + 8lg + e) by two
    // transposing loads each, and the epilogue's x values (8 bytes of row 16it + li)
    u32x4 xa[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int k0 = 32 * kb + 8 * lg;
      const u32x2 lo = lds_tr(sX + (k0 + (li >> 2)) * LDX + 16 * w + 4 * (li & 3));
      const u32x2 hi = lds_tr(sX + (k0 + 4 + (li >> 2)) * LDX + 16 * w + 4 * (li & 3));
      xa[kb] = u32x4{lo[0], lo[1], hi[0], hi[1]};
    }
    u32x2 xe[4];
#pragma unroll
    for (int it = 0; it < 4; ++it) xe[it] = lds64(sX + (16 * it + li) * LDX + 16 * w + 4 * lg);

    // ---- G^T tiles -> M (lower triangle): wave w takes tiles w, w+4, w+8
    {
      f32x4 acc[3];
      int Jt[3], It[3];
      const int ntiles = w < 2 ? 3 : 2;  // tiles w, w+4, w+8 (< 10); wave-uniform
#pragma unroll
      for (int u = 0; u < 3; ++u) {
        const int ti = w + 4 * u < 10 ? w + 4 * u : w;
        // ti -> (Jt, It), It >= Jt: (0,0) (0,1) (0,2) (0,3) (1,1) (1,2) (1,3) (2,2) (2,3) (3,3)
        Jt[u] = ti < 4 ? 0 : (ti < 7 ? 1 : (ti < 9 ? 2 : 3));
        It[u] = ti < 4 ? ti : (ti < 7 ? ti - 3 : (ti < 9 ? ti - 5 : 3));
        acc[u] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int u = 0; u < 3; ++u) {
          if (u == 2 && ntiles < 3) continue;
          const bf16x8 a = as_bf16x8(lds128(sB + (16 * Jt[u] + li) * LDB + 32 * kb + 8 * lg));
          const bf16x8 bb = as_bf16x8(lds128(sC + (16 * It[u] + li) * LDB + 32 * kb + 8 * lg));
          acc[u] = mfma(a, bb, acc[u]);
        }
#pragma unroll
      for (int u = 0; u < 3; ++u) {
        if (u == 2 && ntiles < 3) continue;
        // acc[r] = G[i][j], i = 16It + li, j = 16Jt + 4lg + r
        const int i = 16 * It[u] + li;
        const float csi = sCS[i];
        float m[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int j = 16 * Jt[u] + 4 * lg + r;
          // computed for every lane and selected (the clamp keeps masked entries finite)
          const float v = acc[u][r] * fast_exp2(fminf(csi - sCS[j], 0.0f)) * sDT[j];
          m[r] = j <= i ? v : 0.0f;
        }
        uint32_t* dst = (uint32_t*)(sM + i * LDM + 16 * Jt[u] + 4 * lg);
        dst[0] = pack2(m[0], m[1]);
        dst[1] = pack2(m[2], m[3]);
      }
    }

    load_c(pf, c + 1);
    // ---- Y^T = S_in C^T, columns scaled by exp(cs_i). A operand: the state,
    // k = n in {32kb + 4lg + r} U {32kb + 16 + 4lg + r} (the accumulator layout);
    // B operand: C[i][n] for the same n, two 8-byte pieces of row i.
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
        const uint16_t* cp = sC + (16 * it + li) * LDB + 32 * kb + 4 * lg;
        const u32x2 lo = lds64(cp), hi = lds64(cp + 16);
        yacc[it] = mfma(aop, as_bf16x8(u32x4{lo[0], lo[1], hi[0], hi[1]}), yacc[it]);
      }
    }
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const float ei = sE[16 * it + li];
#pragma unroll
      for (int r = 0; r < 4; ++r) yacc[it][r] *= ei;
    }

    load_x(pf, c + 1);
    // ---- S = exp(cs_last) S + B^T (w x). A operand: B^T rows n = 16nt + li, k = j
    // (transposing loads of B); B operand: w_j x[j][16w + li] from the x^T fragments.
    bf16x8 wxb[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int j0 = 32 * kb + 8 * lg;
      const f32x4 w0 = *(const f32x4*)(sW + j0), w1 = *(const f32x4*)(sW + j0 + 4);
      const u32x4 v = xa[kb];
      wxb[kb] = as_bf16x8(u32x4{pack2(lo_f(v[0]) * w0[0], hi_f(v[0]) * w0[1]),
                                pack2(lo_f(v[1]) * w0[2], hi_f(v[1]) * w0[3]),
                                pack2(lo_f(v[2]) * w1[0], hi_f(v[2]) * w1[1]),
                                pack2(lo_f(v[3]) * w1[2], hi_f(v[3]) * w1[3])});
    }
    const float dec_last = sE[Q - 1];
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) {
#pragma unroll
      for (int r = 0; r < 4; ++r) hacc[nt][r] *= dec_last;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const int k0 = 32 * kb + 8 * lg;
        const u32x2 lo = lds_tr(sB + (k0 + (li >> 2)) * LDB + 16 * nt + 4 * (li & 3));
        const u32x2 hi = lds_tr(sB + (k0 + 4 + (li >> 2)) * LDB + 16 * nt + 4 * (li & 3));
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
      const __amdgpu_buffer_rsrc_t rY = chunk_rsrc(Yb, t0, xz_row);
#pragma unroll
      for (int it = 0; it < 4; ++it) {
        const float xs[4] = {lo_f(xe[it][0]), hi_f(xe[it][0]), lo_f(xe[it][1]), hi_f(xe[it][1])};
        const float zs[4] = {lo_f(zkeep[it][0]), hi_f(zkeep[it][0]), lo_f(zkeep[it][1]), hi_f(zkeep[it][1])};
        float v[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) v[r] = fmaf(Dh, xs[r], yacc[it][r]) * (gate ? silu(zs[r]) : 1.0f);
        const u32x2 out = {pack2(v[0], v[1]), pack2(v[2], v[3])};
        __builtin_amdgcn_raw_buffer_store_b64(out, rY, (int)(e_lane + it * 16 * xz_row), 0, 0);
      }
    }
    // ---- the next chunk's z into the registers the epilogue freed; the next chunk
    // into LDS (past the end: zeros, harmless)
    load_z(zkeep, c + 1);
    stage(pf, c + 1);
    __syncthreads();  // ---- barrier A of chunk c + 1
  }

  // final state, [b, h, p, n]
#pragma unroll
  for (int nt = 0; nt < 8; ++nt) {
    float* hp = k.h_out + ((b * H + h) * P + 16 * w + li) * NS + 16 * nt + 4 * lg;
    *(f32x4*)hp = hacc[nt];
  }
}

bool ssd_chunk_supported(const SSDArgs& a) {
  // buffer offsets are 32-bit: each batch row of x / z / y / B / C must stay below 2^31 bytes
  const int64_t row_x = a.L * a.H * P * 2, row_bc = a.L * a.G * NS * 2;
  return a.bf16 && a.P == P && a.N == NS && a.states == nullptr && a.batch * a.H <= 0x7fffffff &&
         row_x < (int64_t(1) << 31) && row_bc < (int64_t(1) << 31);
}

size_t ssd_chunk_ws(const SSDArgs&) { return 0; }

hipError_t launch_ssd_chunk(const SSDArgs& a, void*, hipStream_t s) {
  if (a.batch == 0) return hipSuccess;
  SsdK k{};
  k.x = (const uint16_t*)a.x; k.dt = (const uint16_t*)a.dt; k.dt_bias = a.dt_bias; k.A_log = a.A_log;
  k.B = (const uint16_t*)a.B; k.C = (const uint16_t*)a.C; k.D = a.D; k.z = (const uint16_t*)a.z;
  k.h0 = a.h0; k.y = (uint16_t*)a.y; k.h_out = a.h_out;
  k.L = a.L; k.H = a.H; k.G = a.G; k.heads_per_group = (int)(a.H / a.G);
  k.nblocks = (int)(a.batch * a.H);
  hipLaunchKernelGGL(ssd_chunk_kernel, dim3((unsigned)k.nblocks), dim3(256), 0, s, k);
  return hipGetLastError();
}

}  // namespace sscan
