// ssd_attention.hip -- the SSD scan's hidden attention map as an optional output.
//
// "Mamba-2" (nnterp encyclopedia), section "The hidden attention": per head the
// scan is a causal linear map over tokens, y_t = sum_s alpha[t, s] x_s + D x_t
// before the gate, with
//     alpha[t, s] = (C_t . B_s) * exp(decays_{s+1} + ... + decays_t) * betas_s   (s <= t)
// and 0 above the diagonal; betas = softplus(dt_raw + dt_bias), decays = betas * A,
// A = -exp(A_log) (section "The mixer's values"); head h reads group h / (H / G).
//
// One workgroup per query token t and batch row. It stages C_t, then walks the
// keys downward from s = t in blocks of 256: first every thread forms one
// C_t . B_s per group, then one thread per head walks the block's keys in
// descending order, keeping the decay sum decays_{s+1} + ... + decays_t in fp64
// (a sum of same-sign terms, formed in the order the definition adds them, with
// no difference of running sums) and writing alpha[b, t, s, h], the heads of one
// key contiguous. The entries above the diagonal are written as zeros. The map
// is [batch, seqlen, seqlen, heads] and is meant for inspection at modest lengths.
#include "device_common.hpp"
#include "mixer_ops.hpp"

namespace sscan {

namespace {

constexpr int kKeys = 256;      // keys per block of the walk (= threads)
constexpr int kMaxHeadsPerThread = 4;

template <typename T>
__global__ __launch_bounds__(256) void ssd_attention_kernel(AttnArgs a) {
  extern __shared__ __attribute__((aligned(16))) float smem[];
  const int64_t L = a.L, H = a.H, N = a.N, G = a.G;
  const int64_t t = blockIdx.x, b = blockIdx.y;
  const int tid = threadIdx.x;
  float* sC = smem;          // [G][N]: C_t
  float* sCB = smem + G * N;  // [G][kKeys]: C_t . B_s for the keys of the block
  const T* Cb = (const T*)a.C + (b * L + t) * G * N;
  for (int64_t e = tid; e < G * N; e += 256) sC[e] = Act<T>::ld(Cb + e);
  const int64_t hpg = H / G;
  // this thread's heads: tid, tid + 256, ...
  double run[kMaxHeadsPerThread];  // decays_{s+1} + ... + decays_t for the next key s
  float A[kMaxHeadsPerThread], bias[kMaxHeadsPerThread];
#pragma unroll
  for (int i = 0; i < kMaxHeadsPerThread; ++i) {
    const int64_t h = tid + 256 * i;
    run[i] = 0.0;
    A[i] = h < H ? -expf(a.A_log[h]) : 0.f;
    bias[i] = h < H ? a.dt_bias[h] : 0.f;
  }
  float* out = a.alpha + (b * L + t) * L * H;  // row t: [s][h]
  for (int64_t hi = t; hi >= 0; hi -= kKeys) {
    const int64_t lo = hi - kKeys + 1 > 0 ? hi - kKeys + 1 : 0;  // keys lo .. hi
    __syncthreads();  // sC staged; the previous block's sCB read
    {
      const int64_t s = lo + tid;
      if (s <= hi) {
        for (int64_t g = 0; g < G; ++g) {
          const T* Bs = (const T*)a.B + ((b * L + s) * G + g) * N;
          float acc = 0.f;
          for (int64_t n = 0; n < N; ++n) acc = fmaf(sC[g * N + n], Act<T>::ld(Bs + n), acc);
          sCB[g * kKeys + tid] = acc;
        }
      }
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kMaxHeadsPerThread; ++i) {
      const int64_t h = tid + 256 * i;
      if (h >= H) continue;
      const int64_t g = h / hpg;
      double r = run[i];
      for (int64_t s = hi; s >= lo; --s) {
        const float beta = softplus(Act<T>::ld((const T*)a.dt + (b * L + s) * H + h) + bias[i]);
        out[s * H + h] = sCB[g * kKeys + (s - lo)] * fast_exp2((float)r * kLog2e) * beta;
        r += (double)beta * (double)A[i];  // the decay of key s joins the sum for keys below it
      }
      run[i] = r;
    }
  }
  // above the diagonal: zeros
  for (int64_t e = (t + 1) * H + tid; e < L * H; e += 256) out[e] = 0.f;
}

}  // namespace

bool ssd_attention_supported(const AttnArgs& a) {
  return a.H <= 256 * kMaxHeadsPerThread && a.G * a.N + a.G * kKeys <= 16384;  // 64 KiB of LDS
}

hipError_t launch_ssd_attention(const AttnArgs& a, hipStream_t s) {
  if (a.batch == 0 || a.L == 0) return hipSuccess;
  const dim3 grid((unsigned)a.L, (unsigned)a.batch), blk(256);
  const size_t lds = (size_t)(a.G * a.N + a.G * kKeys) * sizeof(float);
  if (a.bf16) hipLaunchKernelGGL(ssd_attention_kernel<uint16_t>, grid, blk, lds, s, a);
  else hipLaunchKernelGGL(ssd_attention_kernel<float>, grid, blk, lds, s, a);
  return hipGetLastError();
}

}  // namespace sscan
