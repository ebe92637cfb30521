// launch.hpp -- internal interface between the C ABI (api.cpp) and the kernel launchers.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace sscan {

// Process-wide tuning and test overrides (sscan_set_tuning in sscan.h), read
// when a launch is planned. 0 means the library's own choice.
enum Knob {
  kKnobM1Lanes = 1,          // lanes per channel of the Mamba-1 prompt kernel: 1, 2, 4 or 16
  kKnobSsdSegmentChunks = 2, // chunks per segment of the SSD chunk kernel
  kKnobSsdWorkgroups = 3,    // workgroups of the SSD chunk kernel
  kKnobSsdGiveUp = 4,        // nonzero: every state hand-off wait of the chunk kernel gives up at once
  kKnobSsdHeadsPerWorkgroup = 5,  // 2: two heads per workgroup of the chunk kernel where they share a group
  kKnobSsdF32TokenLoop = 6,  // nonzero: fp32 SSD activations take the token loop, not the fp32 chunk kernel
  kKnobSsdTwoPass = 7,       // SSD chunk kernels: 1 one pass (chained segments), 2 two passes; 0 the plan's choice
  kKnobSsdSplitState = 8,    // nonzero: the bf16 SSD chunk kernel carries the state and w x as two bf16 parts
  kKnobCount = 9
};
int64_t knob(int which);

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
// Shapes the quad-lane kernel takes: state_dim 16, 32 or 64 and channels in whole
// 16-byte pieces (es: bytes per activation).
inline bool m1_quad_ok(int64_t N, int64_t Dc, int64_t es) {
  return (N == 16 || N == 32 || N == 64) && Dc % (16 / es) == 0;
}

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
  size_t ws_cap;  // nonzero: the chunk path's plan keeps its workspace within this (else one pass)
};

// Token-loop SSD (tokenloop.hip): any dtype, state_dim <= 128, per-token states.
size_t ssd_tokenloop_ws(const SSDArgs& a);
hipError_t launch_ssd_tokenloop(const SSDArgs& a, void* ws, hipStream_t s);
hipError_t launch_ssd_step(const SSDArgs& a, hipStream_t s);

// The static device scratch of the entry point that allocates nothing (scratch.hip):
// its size, and its device address on the current device (looked up once per device).
constexpr size_t kScratchBytes = size_t(16) << 20;
hipError_t scratch_ptr(void** out);

// MFMA chunk SSD (ssd_chunk.hip): bf16 or fp32, head_dim 64 times a power of two, state_dim 64..128,
// no per-token states.
bool ssd_chunk_supported(const SSDArgs& a);
size_t ssd_chunk_ws(const SSDArgs& a);
hipError_t launch_ssd_chunk(const SSDArgs& a, void* ws, hipStream_t s);

}  // namespace sscan
