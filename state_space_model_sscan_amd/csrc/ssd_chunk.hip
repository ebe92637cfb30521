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
// whole sequence, and it produces those 16 columns of y. Per chunk:
//   1. stage B, C (row-major), B^T and x in LDS as bf16; cumulative decay of dt;
//   2. G^T = B C^T on MFMA (10 lower-triangular 16x16 tiles shared out over the
//      waves), masked and scaled into M[i, j] = G[i, j] exp(cs_i - cs_j) dt_j
//      (bf16, in LDS);
//   3. Y = diag(exp(cs)) (C S_in^T): the B operand comes straight from the state
//      accumulators, converted to bf16;
//   4. Y += M X;
//   5. S = exp(cs_last) S + B^T (w X), w_j = exp(cs_last - cs_j) dt_j;
//   6. y = Y + D x, times silu(z), stored as bf16.
// The global loads of chunk c+1 are in flight while chunk c is computed.
// MFMA: v_mfma_f32_16x16x32_bf16. Operand layouts (verified on gfx950):
// A[16 x 32]: lane l holds row l%16, k = 8*(l/16) .. +8; B[32 x 16]: lane l
// holds column l%16, the same k; D[16 x 16]: lane l holds rows 4*(l/16) + r,
// column l%16. Any assignment of k to (lane group, element) works as long as
// A and B use the same one; step 3 uses k = {4g+r} U {16+4g+r} to match the
// accumulator layout of the state.
#include "device_common.hpp"
#include "launch.hpp"

namespace sscan {

namespace {

constexpr int Q = 64;      // tokens per chunk
constexpr int P = 64;      // head_dim
constexpr int NS = 128;    // state_dim
constexpr int LDB = NS + 8;   // row pitch (bf16) of sB, sC
constexpr int LDBT = Q + 8;   // row pitch of sBT (one row per state entry)
constexpr int LDX = P + 8;    // row pitch of sX
constexpr int LDM = Q + 8;    // row pitch of sM

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

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

__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  return (uint32_t)f32_to_bf16(lo) | ((uint32_t)f32_to_bf16(hi) << 16);
}

// chunk-ahead global loads of one thread (16-byte pieces; zeros past the sequence end)
struct Prefetch {
  u32x4 b[4], c[4], x[2];
  float dt;
};

}  // namespace

__global__ __launch_bounds__(256, 2) void ssd_chunk_kernel(SsdK k) {
  __shared__ __attribute__((aligned(16))) uint16_t sB[Q * LDB];
  __shared__ __attribute__((aligned(16))) uint16_t sC[Q * LDB];
  __shared__ __attribute__((aligned(16))) uint16_t sBT[NS * LDBT];
  __shared__ __attribute__((aligned(16))) uint16_t sX[Q * LDX];
  __shared__ __attribute__((aligned(16))) uint16_t sM[Q * LDM];
  __shared__ float sDT[Q], sCS[Q], sW[Q], sE[Q];

  // block -> (batch, head): consecutive heads of one batch row share an XCD (and its L2)
  int lin = blockIdx.x;
  if (k.nblocks % 8 == 0) lin = (blockIdx.x % 8) * (k.nblocks / 8) + blockIdx.x / 8;
  const int64_t b = lin / k.H, h = lin % k.H;
  const int64_t g = h / k.heads_per_group;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, li = l & 15, lg = l >> 4;
  const int64_t L = k.L, H = k.H, G = k.G;
  const float A2 = -expf(k.A_log[h]) * kLog2e;  // decay per unit step, exp2 domain
  const float bias = k.dt_bias[h];
  const float Dh = k.D[h];
  const int p_own = 16 * w + li;  // the head_dim column this lane holds in D layouts

  // state slice: hacc[Nt][r] = S[p = 16w + li][n = 16Nt + 4lg + r]
  f32x4 hacc[8];
#pragma unroll
  for (int nt = 0; nt < 8; ++nt) {
    if (k.h0) {
      const float* hp = k.h0 + ((b * H + h) * P + p_own) * NS + 16 * nt + 4 * lg;
      hacc[nt] = *(const f32x4*)hp;
    } else {
      hacc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  }
  // the tiles of M above the diagonal block row stay zero
  for (int e = tid; e < Q * LDM; e += 256) sM[e] = 0;

  const int64_t nchunks = (L + Q - 1) / Q;
  auto load_chunk = [&](Prefetch& pf, int64_t c) {
    const int64_t t0 = c * Q;
#pragma unroll
    for (int it = 0; it < 4; ++it) {  // B, C: 64 rows x 16 pieces
      const int idx = tid + 256 * it, row = idx >> 4, piece = idx & 15;
      const int64_t t = t0 + row;
      const bool ok = c < nchunks && t < L;
      const int64_t off = ((b * L + (ok ? t : 0)) * G + g) * NS + piece * 8;
      pf.b[it] = ok ? *(const u32x4*)(k.B + off) : u32x4{0, 0, 0, 0};
      pf.c[it] = ok ? *(const u32x4*)(k.C + off) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int it = 0; it < 2; ++it) {  // x: 64 rows x 8 pieces
      const int idx = tid + 256 * it, row = idx >> 3, piece = idx & 7;
      const int64_t t = t0 + row;
      const bool ok = c < nchunks && t < L;
      const int64_t off = ((b * L + (ok ? t : 0)) * H + h) * P + piece * 8;
      pf.x[it] = ok ? *(const u32x4*)(k.x + off) : u32x4{0, 0, 0, 0};
    }
    if (tid < Q) {
      const int64_t t = t0 + tid;
      const bool ok = c < nchunks && t < L;
      pf.dt = ok ? bf16_to_f32(k.dt[(b * L + t) * H + h]) : 0.0f;
    }
  };

  Prefetch pf;
  load_chunk(pf, 0);

  for (int64_t c = 0; c < nchunks; ++c) {
    const int64_t t0 = c * Q;
    const int nt_valid = (int)min((int64_t)Q, L - t0);
    __syncthreads();  // the previous chunk is done with every LDS buffer
    // ---- 1. stage
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int idx = tid + 256 * it, row = idx >> 4, piece = idx & 15;
      *(u32x4*)(sB + row * LDB + piece * 8) = pf.b[it];
      *(u32x4*)(sC + row * LDB + piece * 8) = pf.c[it];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t wv = pf.b[it][e >> 1];
        sBT[(piece * 8 + e) * LDBT + row] = (uint16_t)((e & 1) ? (wv >> 16) : (wv & 0xffffu));
      }
    }
#pragma unroll
    for (int it = 0; it < 2; ++it) {
      const int idx = tid + 256 * it, row = idx >> 3, piece = idx & 7;
      *(u32x4*)(sX + row * LDX + piece * 8) = pf.x[it];
    }
    if (tid < Q) {  // wave 0: steps and their inclusive cumulative sum (exp2 domain)
      const bool ok = tid < nt_valid;
      const float dtv = ok ? softplus(pf.dt + bias) : 0.0f;  // a token past the end is a zero step
      float cs = dtv * A2;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const float o = __shfl_up(cs, off, 64);
        if (tid >= off) cs += o;
      }
      const float cs_last = __shfl(cs, 63, 64);
      sDT[tid] = dtv;
      sCS[tid] = cs;
      sE[tid] = fast_exp2(cs);
      sW[tid] = fast_exp2(cs_last - cs) * dtv;
    }
    // z of this chunk for the epilogue (rows i = 16It + 4lg + r, column p_own)
    float zv[4][4];
    if (k.z) {
#pragma unroll
      for (int it = 0; it < 4; ++it)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int i = 16 * it + 4 * lg + r;
          const int64_t t = t0 + (i < nt_valid ? i : 0);
          zv[it][r] = bf16_to_f32(k.z[((b * L + t) * H + h) * P + p_own]);
        }
    }
    // the next chunk's loads run during this chunk's compute
    load_chunk(pf, c + 1);
    __syncthreads();

    // ---- 2. G^T tiles -> M (lower triangle), shared out over the waves
    for (int ti = w; ti < 10; ti += 4) {
      // ti -> (Jt, It), It >= Jt: (0,0) (0,1) (0,2) (0,3) (1,1) (1,2) (1,3) (2,2) (2,3) (3,3)
      const int Jt = ti < 4 ? 0 : (ti < 7 ? 1 : (ti < 9 ? 2 : 3));
      const int It = ti < 4 ? ti : (ti < 7 ? ti - 3 : (ti < 9 ? ti - 5 : 3));
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const bf16x8 a = as_bf16x8(lds128(sB + (16 * Jt + li) * LDB + 32 * kb + 8 * lg));
        const bf16x8 bb = as_bf16x8(lds128(sC + (16 * It + li) * LDB + 32 * kb + 8 * lg));
        acc = mfma(a, bb, acc);
      }
      // acc[r] = G[i][j], i = 16It + li, j = 16Jt + 4lg + r
      const int i = 16 * It + li;
      const float csi = sCS[i];
      float m[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int j = 16 * Jt + 4 * lg + r;
        m[r] = j <= i ? acc[r] * fast_exp2(csi - sCS[j]) * sDT[j] : 0.0f;
      }
      uint32_t* dst = (uint32_t*)(sM + i * LDM + 16 * Jt + 4 * lg);
      dst[0] = pack2(m[0], m[1]);
      dst[1] = pack2(m[2], m[3]);
    }

    // ---- x of this wave's 16 columns as B operands: X[j][p_own], j = 32kb + 8lg + e
    float xw[2][8];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int e = 0; e < 8; ++e) xw[kb][e] = bf16_to_f32(sX[(32 * kb + 8 * lg + e) * LDX + p_own]);

    // ---- 3. Y = C S_in^T (before the state moves on), rows scaled by exp(cs_i)
    f32x4 yacc[4];
#pragma unroll
    for (int it = 0; it < 4; ++it) yacc[it] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      // B operand: S[p_own][n] for n in {32kb + 4lg + r} U {32kb + 16 + 4lg + r}
      u32x4 sv;
      sv[0] = pack2(hacc[2 * kb][0], hacc[2 * kb][1]);
      sv[1] = pack2(hacc[2 * kb][2], hacc[2 * kb][3]);
      sv[2] = pack2(hacc[2 * kb + 1][0], hacc[2 * kb + 1][1]);
      sv[3] = pack2(hacc[2 * kb + 1][2], hacc[2 * kb + 1][3]);
      const bf16x8 bop = as_bf16x8(sv);
#pragma unroll
      for (int it = 0; it < 4; ++it) {
        const uint16_t* cp = sC + (16 * it + li) * LDB + 32 * kb + 4 * lg;
        const uint2 lo = *(const uint2*)cp;
        const uint2 hi = *(const uint2*)(cp + 16);
        const u32x4 av = {lo.x, lo.y, hi.x, hi.y};
        yacc[it] = mfma(as_bf16x8(av), bop, yacc[it]);
      }
    }
#pragma unroll
    for (int it = 0; it < 4; ++it)
#pragma unroll
      for (int r = 0; r < 4; ++r) yacc[it][r] *= sE[16 * it + 4 * lg + r];

    __syncthreads();  // M complete

    // ---- 4. Y += M X
    bf16x8 xop[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      u32x4 v;
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = pack2(xw[kb][2 * e], xw[kb][2 * e + 1]);
      xop[kb] = as_bf16x8(v);
    }
#pragma unroll
    for (int it = 0; it < 4; ++it) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        if (kb == 1 && it < 2) continue;  // M[i][j] = 0 for j >= 32 when i < 32
        const bf16x8 a = as_bf16x8(lds128(sM + (16 * it + li) * LDM + 32 * kb + 8 * lg));
        yacc[it] = mfma(a, xop[kb], yacc[it]);
      }
    }

    // ---- 5. S = exp(cs_last) S + B^T (w X)
    const float dec_last = sE[Q - 1];
    bf16x8 wxop[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      u32x4 v;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int j = 32 * kb + 8 * lg + 2 * e;
        v[e] = pack2(xw[kb][2 * e] * sW[j], xw[kb][2 * e + 1] * sW[j + 1]);
      }
      wxop[kb] = as_bf16x8(v);
    }
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) {
#pragma unroll
      for (int r = 0; r < 4; ++r) hacc[nt][r] *= dec_last;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const bf16x8 a = as_bf16x8(lds128(sBT + (16 * nt + li) * LDBT + 32 * kb + 8 * lg));
        hacc[nt] = mfma(a, wxop[kb], hacc[nt]);
      }
    }

    // ---- 6. epilogue
#pragma unroll
    for (int it = 0; it < 4; ++it)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = 16 * it + 4 * lg + r;
        if (i < nt_valid) {
          float yv = yacc[it][r] + Dh * bf16_to_f32(sX[i * LDX + p_own]);
          if (k.z) yv *= silu(zv[it][r]);
          k.y[((b * L + t0 + i) * H + h) * P + p_own] = f32_to_bf16(yv);
        }
      }
  }

  // final state, [b, h, p, n]
#pragma unroll
  for (int nt = 0; nt < 8; ++nt) {
    float* hp = k.h_out + ((b * H + h) * P + p_own) * NS + 16 * nt + 4 * lg;
    *(f32x4*)hp = hacc[nt];
  }
}

bool ssd_chunk_supported(const SSDArgs& a) {
  return a.bf16 && a.P == P && a.N == NS && a.states == nullptr && a.batch * a.H <= 0x7fffffff;
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
