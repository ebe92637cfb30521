// mixer_ops.hip -- the steps next to the scan: causal depthwise conv1d + silu in
// front of it, and the gated RMS norm after the Mamba-2 SSD.
//
// conv1d + silu ("Mamba-2", nnterp encyclopedia, section "The block, in order":
// x, B, C = silu(conv1d(xBC)), causal, width 4; "Mamba", tokentrails lineage,
// section "Code": depthwise, width 4): one lane per channel (coalesced over
// channels) walks a block of 64 tokens with the last W-1 inputs in registers;
// the W-1 inputs before a block come from x itself or, before the call's first
// token, from the carried conv state.
//
// gated RMS norm ("Mamba-2", section "The block, in order" and the note under
// it): g = y * silu(z) normalised over the whole width of the row, times the
// norm's weight. One workgroup per row: pass 1 sums g^2 (wave DPP/shuffle
// reduction, then across the 4 waves in LDS), pass 2 re-reads the row (L2-hot)
// and writes g * rsqrt(mean + eps) * weight.
#include "device_common.hpp"
#include "mixer_ops.hpp"

namespace sscan {

namespace {

constexpr int kConvTokens = 64;

template <typename T, int W>
__global__ __launch_bounds__(256) void conv1d_silu_kernel(ConvArgs a) {
  const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (c >= a.Dc) return;
  const int64_t b = blockIdx.z;
  const int64_t t0 = (int64_t)blockIdx.y * kConvTokens;
  const int64_t t1 = min(a.L, t0 + kConvTokens);
  const T* x = (const T*)a.x;
  T* out = (T*)a.out;
  float wt[W];
#pragma unroll
  for (int kk = 0; kk < W; ++kk) wt[kk] = a.weight[c * W + kk];
  const float bias = a.bias ? a.bias[c] : 0.0f;
  float hist[W > 1 ? W - 1 : 1];  // inputs at t0-W+1 .. t0-1, oldest first
#pragma unroll
  for (int kk = 0; kk < W - 1; ++kk) {
    const int64_t pos = t0 - (W - 1) + kk;
    if (pos >= 0)
      hist[kk] = Act<T>::ld(x + (b * a.L + pos) * a.Dc + c);
    else
      hist[kk] = a.state_in ? a.state_in[(b * a.Dc + c) * (W - 1) + (W - 1 + pos)] : 0.0f;
  }
  for (int64_t t = t0; t < t1; ++t) {
    const float xt = Act<T>::ld(x + (b * a.L + t) * a.Dc + c);
    float acc = bias;
#pragma unroll
    for (int kk = 0; kk < W - 1; ++kk) acc = fmaf(wt[kk], hist[kk], acc);
    acc = fmaf(wt[W - 1], xt, acc);
    Act<T>::st(out + (b * a.L + t) * a.Dc + c, silu(acc));
#pragma unroll
    for (int kk = 0; kk + 1 < W - 1; ++kk) hist[kk] = hist[kk + 1];
    if (W > 1) hist[W > 1 ? W - 2 : 0] = xt;
  }
}

// conv_state_out = the last W-1 inputs of [state_in, x] (oldest first).
template <typename T>
__global__ __launch_bounds__(256) void conv_state_kernel(ConvArgs a) {
  const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (c >= a.Dc) return;
  const int64_t b = blockIdx.y;
  const int W = (int)a.W;
  const T* x = (const T*)a.x;
  for (int kk = 0; kk < W - 1; ++kk) {
    const int64_t pos = a.L - (W - 1) + kk;
    float v;
    if (pos >= 0)
      v = Act<T>::ld(x + (b * a.L + pos) * a.Dc + c);
    else
      v = a.state_in ? a.state_in[(b * a.Dc + c) * (W - 1) + (W - 1 + pos)] : 0.0f;
    a.state_out[(b * a.Dc + c) * (W - 1) + kk] = v;
  }
}

__device__ __forceinline__ float block_sum_256(float v, float* red) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  const float s = red[0] + red[1] + red[2] + red[3];
  __syncthreads();
  return s;
}

template <typename T>
__global__ __launch_bounds__(256) void gated_rmsnorm_kernel(NormArgs a) {
  __shared__ float red[4];
  const int64_t row = blockIdx.x;
  const T* y = (const T*)a.y + row * a.width;
  const T* z = (const T*)a.z + row * a.width;
  T* out = (T*)a.out + row * a.width;
  float ss = 0.0f;
  for (int64_t i = threadIdx.x; i < a.width; i += 256) {
    const float g = Act<T>::ld(y + i) * silu(Act<T>::ld(z + i));
    ss = fmaf(g, g, ss);
  }
  const float total = block_sum_256(ss, red);
  const float inv = 1.0f / sqrtf(total / (float)a.width + a.eps);
  for (int64_t i = threadIdx.x; i < a.width; i += 256) {
    const float g = Act<T>::ld(y + i) * silu(Act<T>::ld(z + i));
    Act<T>::st(out + i, g * inv * a.weight[i]);
  }
}

template <typename T>
void launch_conv_t(const ConvArgs& a, hipStream_t s) {
  const unsigned cb = (unsigned)((a.Dc + 255) / 256);
  if (a.L > 0) {
    const dim3 grid(cb, (unsigned)((a.L + kConvTokens - 1) / kConvTokens), (unsigned)a.batch);
    switch (a.W) {
      case 1: hipLaunchKernelGGL((conv1d_silu_kernel<T, 1>), grid, dim3(256), 0, s, a); break;
      case 2: hipLaunchKernelGGL((conv1d_silu_kernel<T, 2>), grid, dim3(256), 0, s, a); break;
      case 3: hipLaunchKernelGGL((conv1d_silu_kernel<T, 3>), grid, dim3(256), 0, s, a); break;
      case 4: hipLaunchKernelGGL((conv1d_silu_kernel<T, 4>), grid, dim3(256), 0, s, a); break;
      case 5: hipLaunchKernelGGL((conv1d_silu_kernel<T, 5>), grid, dim3(256), 0, s, a); break;
      case 6: hipLaunchKernelGGL((conv1d_silu_kernel<T, 6>), grid, dim3(256), 0, s, a); break;
      case 7: hipLaunchKernelGGL((conv1d_silu_kernel<T, 7>), grid, dim3(256), 0, s, a); break;
      default: hipLaunchKernelGGL((conv1d_silu_kernel<T, 8>), grid, dim3(256), 0, s, a); break;
    }
  }
  if (a.state_out && a.W > 1)
    hipLaunchKernelGGL(conv_state_kernel<T>, dim3(cb, (unsigned)a.batch), dim3(256), 0, s, a);
}

}  // namespace

hipError_t launch_conv1d_silu(const ConvArgs& a, hipStream_t s) {
  if (a.batch == 0) return hipSuccess;
  if (a.bf16) launch_conv_t<uint16_t>(a, s);
  else launch_conv_t<float>(a, s);
  return hipGetLastError();
}

hipError_t launch_gated_rmsnorm(const NormArgs& a, hipStream_t s) {
  if (a.rows == 0) return hipSuccess;
  if (a.bf16) hipLaunchKernelGGL(gated_rmsnorm_kernel<uint16_t>, dim3((unsigned)a.rows), dim3(256), 0, s, a);
  else hipLaunchKernelGGL(gated_rmsnorm_kernel<float>, dim3((unsigned)a.rows), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace sscan
