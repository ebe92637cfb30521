// launch.hpp -- internal interface between the C ABI (api.cpp) and the kernel launchers.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace sscan {

struct Mamba1Args {
  int64_t batch, L, Dc, N, G;
  bool bf16;
  float bc_eps;  // <= 0: off
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
};

// Launch plan of a prompt scan (a pure function of the shape): lanes per channel
// and the cut of the sequence into slices (workspace holds the slice carries).
struct Mamba1Plan {
  int64_t nslices;
  int64_t slice_len;
  size_t ws_bytes;
  int64_t lanes_per_channel;
};
Mamba1Plan mamba1_plan(int64_t batch, int64_t L, int64_t Dc, int64_t N, int64_t G, int64_t es);  // 0 lanes: token loop
Mamba1Plan tokenloop_plan(int64_t batch, int64_t L, int64_t Dc, int64_t N);  // token-loop kernel
hipError_t launch_m1_fast(const Mamba1Args& a, const Mamba1Plan& plan, const float* ws_h, const float* ws_sdt,
                          hipStream_t s);

hipError_t launch_mamba1_fwd(const Mamba1Args& a, const Mamba1Plan& plan, void* ws, hipStream_t s);
hipError_t launch_mamba1_step(const Mamba1Args& a, hipStream_t s);

struct SSDArgs {
  int64_t batch, L, H, P, N, G, chunk;
  bool bf16;
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
};

// Token-loop SSD (tokenloop.hip): any dtype, state_dim <= 128, per-token states.
size_t ssd_tokenloop_ws(const SSDArgs& a);
hipError_t launch_ssd_tokenloop(const SSDArgs& a, void* ws, hipStream_t s);
hipError_t launch_ssd_step(const SSDArgs& a, hipStream_t s);

// MFMA chunk SSD (ssd_chunk.hip): bf16, head_dim 64, state_dim 128, no per-token states.
bool ssd_chunk_supported(const SSDArgs& a);
size_t ssd_chunk_ws(const SSDArgs& a);
hipError_t launch_ssd_chunk(const SSDArgs& a, void* ws, hipStream_t s);

}  // namespace sscan
