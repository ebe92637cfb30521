// tokenloop.hip -- host side of the token-loop scan: slicing plan and launches.
// The kernels are in tokenloop_impl.hpp, instantiated in tl_*.hip.
#include "tokenloop_impl.hpp"

namespace sscan {

extern template void dispatch_scan<float, false>(const TLK&, int64_t, bool, bool, hipStream_t);
extern template void dispatch_scan<float, true>(const TLK&, int64_t, bool, bool, hipStream_t);
extern template void dispatch_scan<uint16_t, false>(const TLK&, int64_t, bool, bool, hipStream_t);
extern template void dispatch_scan<uint16_t, true>(const TLK&, int64_t, bool, bool, hipStream_t);
extern template void dispatch_pass1<float, false>(const TLK&, int64_t, hipStream_t);
extern template void dispatch_pass1<uint16_t, false>(const TLK&, int64_t, hipStream_t);
extern template void dispatch_step<float, false>(const TLK&, int64_t, bool, hipStream_t);
extern template void dispatch_step<float, true>(const TLK&, int64_t, bool, hipStream_t);
extern template void dispatch_step<uint16_t, false>(const TLK&, int64_t, bool, hipStream_t);
extern template void dispatch_step<uint16_t, true>(const TLK&, int64_t, bool, hipStream_t);

// seqlen 0: the state passes through (or is zero).
__global__ void copy_or_zero_kernel(const float* src, float* dst, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) dst[i] = src ? src[i] : 0.0f;
}

// Slices for the token-loop prompt scan (a pure function of the shape).
Mamba1Plan tokenloop_plan(int64_t batch, int64_t L, int64_t Dc, int64_t N) {
  Mamba1Plan p{1, L > 0 ? L : 1, 0, 1};
  const int64_t lanes = N > 32 ? 16 : 1;  // tokenloop_group_kernel above 32 states
  const int64_t waves = batch * ((Dc * lanes + 63) / 64);
  // two waves per SIMD on 256 CUs x 4 SIMDs; four for the 16-lane kernel, whose
  // slices are short enough that more of them shorten both passes (four waves per
  // SIMD is also all its LDS lets a unit hold). As many slices as keep the grid
  // within that: a grid a little larger than what the GPU holds at once runs a
  // second, mostly idle round (fp32 SSD at the Mamba-2 2.7B shape, one batch row:
  // 5120 waves took 2.87 ms, 3840 waves 2.40 ms).
  const int64_t target = lanes == 16 ? 4096 : 2048;
  int64_t ns = waves > 0 ? std::max<int64_t>(target / waves, 1) : 1;
  const int64_t max_ns = L / 64 > 1 ? L / 64 : 1;  // slices of at least 64 tokens
  if (ns > max_ns) ns = max_ns;
  if (ns < 1) ns = 1;
  if (ns > 1) {
    int64_t len = (L + ns - 1) / ns;
    len = (len + 63) / 64 * 64;
    ns = (L + len - 1) / len;
    p.slice_len = len;
  }
  p.nslices = ns;
  p.ws_bytes = ns > 1 ? (size_t)(batch * ns * Dc * (N + 1)) * sizeof(float) : 0;
  return p;
}

static void run_tokenloop(TLK k, int64_t batch, bool bf16, bool ssd, bool gate, bool states,
                          const Mamba1Plan& plan, void* ws, hipStream_t s) {
  k.nslices = (int)plan.nslices;
  k.slice_len = (int)plan.slice_len;
  if (plan.nslices > 1) {
    k.ws_h = (float*)ws;
    k.ws_sdt = (float*)ws + batch * plan.nslices * k.Dc * k.N;
  }
  if (bf16) {
    if (ssd) dispatch_scan<uint16_t, true>(k, batch, gate, states, s);
    else dispatch_scan<uint16_t, false>(k, batch, gate, states, s);
  } else {
    if (ssd) dispatch_scan<float, true>(k, batch, gate, states, s);
    else dispatch_scan<float, false>(k, batch, gate, states, s);
  }
}

static TLK make_k(const void* x, const void* dt, const float* dt_bias, const float* A_log, const void* B,
                  const void* C, const float* D, const void* z, const float* h0, void* y, float* h_out,
                  float* states) {
  TLK k{};
  k.x = x; k.dt = dt; k.dt_bias = dt_bias; k.A_log = A_log; k.B = B; k.C = C;
  k.D = D; k.z = z; k.h0 = h0; k.y = y; k.h_out = h_out; k.states = states;
  return k;
}

static hipError_t zero_length(const float* h0, float* h_out, int64_t nst, hipStream_t s) {
  if (nst > 0)
    hipLaunchKernelGGL(copy_or_zero_kernel, dim3((unsigned)((nst + 255) / 256)), dim3(256), 0, s, h0, h_out,
                       nst);
  return hipGetLastError();
}

// Mamba-1 prompt plan. With state_dim 16, 32 or 64: the quad-lane kernel (4
// lanes per channel) when its grid still puts two waves on every one of the 1024
// SIMDs (it spends fewer VALU instructions per state update), else the
// row-per-channel kernel (16 lanes per channel, channels in groups of 4), which
// at the Mamba-130m width keeps three waves per SIMD where four lanes would leave
// a quarter of the SIMDs empty. Other shapes take K = 1, 2 or 4 lanes per channel
// of the general kernel, the smallest K that puts two waves on each SIMD. Slices
// (two-pass carry) only when the grid still has fewer than 512 waves on a long
// sequence.
Mamba1Plan mamba1_plan(int64_t batch, int64_t L, int64_t Dc, int64_t N, int64_t G, int64_t es) {
  // a batch row (of x/dt/z/y, or of B/C) that the 32-bit buffer offsets of the
  // fast kernels cannot span: token-loop kernel
  // or more than 64 states (the fast kernels hold at most 64 per channel): the
  // token-loop kernel
  if (L * Dc * es >= (int64_t(1) << 31) || L * G * N * es >= (int64_t(1) << 31) || N > 64) {
    Mamba1Plan t = tokenloop_plan(batch, L, Dc, N);
    t.lanes_per_channel = 0;
    return t;
  }
  Mamba1Plan p{1, L > 0 ? L : 1, 0, 1};
  auto waves = [&](int64_t K) { return batch * ((Dc * K + 63) / 64); };
  // the row-per-channel kernel (16 lanes) takes state_dim 16, 32 or 64 and
  // channels in whole groups of 4
  const bool row_ok = (N == 16 || N == 32 || N == 64) && Dc % 4 == 0;
  const bool quad_ok = m1_quad_ok(N, Dc, es);
  int64_t K = N > 32 ? 2 : 1;  // 64 states in one lane would spill
  while (K < 4 && waves(K) < 2048) K *= 2;
  if (quad_ok && waves(4) >= 2048) K = 4;
  else if (row_ok) K = 16;
  {  // tuning override: 1, 2, 4 or 16 lanes per channel
    const int64_t v = knob(kKnobM1Lanes);
    if ((v == 1 && N <= 32) || v == 2 || v == 4 || (v == 16 && row_ok)) K = v;
  }
  p.lanes_per_channel = K;
  const int64_t w = waves(K);
  if (w > 0 && w < 512 && L >= 1024) {
    int64_t ns = (1024 + w - 1) / w;
    if (ns > L / 512) ns = L / 512;
    if (ns > 1) {
      int64_t len = (L + ns - 1) / ns;
      len = (len + 63) / 64 * 64;
      ns = (L + len - 1) / len;
      p.nslices = ns;
      p.slice_len = len;
    }
  }
  p.ws_bytes = p.nslices > 1 ? (size_t)(batch * p.nslices * Dc * (N + 1)) * sizeof(float) : 0;
  return p;
}

hipError_t launch_mamba1_fwd(const Mamba1Args& a, const Mamba1Plan& plan, void* ws, hipStream_t s) {
  if (a.L == 0 || a.batch == 0) return zero_length(a.h0, a.h_out, a.batch * a.Dc * a.N, s);
  if (plan.lanes_per_channel == 0) {  // the token-loop kernel, both passes
    TLK k = make_k(a.x, a.dt, a.dt_bias, a.A_log, a.B, a.C, a.D, a.z, a.h0, a.y, a.h_out, a.states);
    k.L = a.L; k.Dc = a.Dc; k.N = (int)a.N; k.G = (int)a.G; k.per_group = a.Dc / a.G;
    k.bc_eps = a.bc_eps; k.H = a.Dc; k.P = 1;
    run_tokenloop(k, a.batch, a.bf16, false, a.z != nullptr, a.states != nullptr, plan, ws, s);
    return hipGetLastError();
  }
  const float* ws_h = nullptr;
  const float* ws_sdt = nullptr;
  if (plan.nslices > 1) {
    TLK k = make_k(a.x, a.dt, a.dt_bias, a.A_log, a.B, a.C, a.D, a.z, a.h0, a.y, a.h_out, a.states);
    k.L = a.L; k.Dc = a.Dc; k.N = (int)a.N; k.G = (int)a.G; k.per_group = a.Dc / a.G;
    k.bc_eps = a.bc_eps; k.H = a.Dc; k.P = 1;
    k.nslices = (int)plan.nslices; k.slice_len = (int)plan.slice_len;
    k.ws_h = (float*)ws;
    k.ws_sdt = (float*)ws + a.batch * plan.nslices * a.Dc * a.N;
    if (a.bf16) dispatch_pass1<uint16_t, false>(k, a.batch, s);
    else dispatch_pass1<float, false>(k, a.batch, s);
    ws_h = k.ws_h;
    ws_sdt = k.ws_sdt;
  }
  return launch_m1_fast(a, plan, ws_h, ws_sdt, s);
}

hipError_t launch_mamba1_step(const Mamba1Args& a, hipStream_t s) {
  if (a.batch == 0) return hipSuccess;
  TLK k = make_k(a.x, a.dt, a.dt_bias, a.A_log, a.B, a.C, a.D, a.z, a.h0, a.y, a.h_out, nullptr);
  k.L = 1; k.Dc = a.Dc; k.N = (int)a.N; k.G = (int)a.G; k.per_group = a.Dc / a.G;
  k.bc_eps = a.bc_eps; k.H = a.Dc; k.P = 1; k.nslices = 1; k.slice_len = 1;
  if (a.bf16) dispatch_step<uint16_t, false>(k, a.batch, a.z != nullptr, s);
  else dispatch_step<float, false>(k, a.batch, a.z != nullptr, s);
  return hipGetLastError();
}

// SSD through the token loop (any dtype, state_dim up to 128, per-token states).
size_t ssd_tokenloop_ws(const SSDArgs& a) { return tokenloop_plan(a.batch, a.L, a.H * a.P, a.N).ws_bytes; }

hipError_t launch_ssd_tokenloop(const SSDArgs& a, void* ws, hipStream_t s) {
  const int64_t Dc = a.H * a.P;
  if (a.L == 0 || a.batch == 0) return zero_length(a.h0, a.h_out, a.batch * Dc * a.N, s);
  TLK k = make_k(a.x, a.dt, a.dt_bias, a.A_log, a.B, a.C, a.D, a.z, a.h0, a.y, a.h_out, a.states);
  k.L = a.L; k.Dc = Dc; k.N = (int)a.N; k.G = (int)a.G; k.per_group = Dc / a.G;
  k.bc_eps = 0.0f; k.H = a.H; k.P = a.P;
  run_tokenloop(k, a.batch, a.bf16, true, a.z != nullptr, a.states != nullptr, tokenloop_plan(a.batch, a.L, Dc, a.N),
                ws, s);
  return hipGetLastError();
}

hipError_t launch_ssd_step(const SSDArgs& a, hipStream_t s) {
  if (a.batch == 0) return hipSuccess;
  const int64_t Dc = a.H * a.P;
  TLK k = make_k(a.x, a.dt, a.dt_bias, a.A_log, a.B, a.C, a.D, a.z, a.h0, a.y, a.h_out, nullptr);
  k.L = 1; k.Dc = Dc; k.N = (int)a.N; k.G = (int)a.G; k.per_group = Dc / a.G;
  k.bc_eps = 0.0f; k.H = a.H; k.P = a.P; k.nslices = 1; k.slice_len = 1;
  if (a.bf16) dispatch_step<uint16_t, true>(k, a.batch, a.z != nullptr, s);
  else dispatch_step<float, true>(k, a.batch, a.z != nullptr, s);
  return hipGetLastError();
}

}  // namespace sscan
