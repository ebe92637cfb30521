// mixer_ops.hpp -- internal interface of the conv1d + silu and gated RMS norm kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sscan {

struct ConvArgs {
  int64_t batch, L, Dc, W;
  bool bf16;
  const void* x;
  const float* weight;
  const float* bias;
  const float* state_in;
  void* out;
  float* state_out;
};
hipError_t launch_conv1d_silu(const ConvArgs& a, hipStream_t s);

struct NormArgs {
  int64_t rows, width;
  bool bf16;
  float eps;
  const void* y;
  const void* z;
  const float* weight;
  void* out;
};
hipError_t launch_gated_rmsnorm(const NormArgs& a, hipStream_t s);

struct AttnArgs {
  int64_t batch, L, H, N, G;
  bool bf16;
  const void* dt;
  const float* dt_bias;
  const float* A_log;
  const void* B;
  const void* C;
  float* alpha;
  double* ws_P;     // [batch, H, L]: decays_0 + ... + decays_t, times log2(e)
  float* ws_beta;   // [batch, H, L]: betas
};
bool ssd_attention_supported(const AttnArgs& a);
size_t ssd_attention_ws(const AttnArgs& a);
hipError_t launch_ssd_attention(const AttnArgs& a, hipStream_t s);

}  // namespace sscan
