// m1_fast.hip -- host launch of the Mamba-1 prompt kernel (m1_fast_impl.hpp).
#include "m1_quad_impl.hpp"

namespace sscan {

extern template void launch_m1_quad_np<float, 16>(const M1F&, bool, bool, dim3, hipStream_t);
extern template void launch_m1_quad_np<float, 32>(const M1F&, bool, bool, dim3, hipStream_t);
extern template void launch_m1_quad_np<float, 64>(const M1F&, bool, bool, dim3, hipStream_t);
extern template void launch_m1_quad_np<uint16_t, 16>(const M1F&, bool, bool, dim3, hipStream_t);
extern template void launch_m1_quad_np<uint16_t, 32>(const M1F&, bool, bool, dim3, hipStream_t);
extern template void launch_m1_quad_np<uint16_t, 64>(const M1F&, bool, bool, dim3, hipStream_t);

extern template void launch_m1_np<float, 16>(const M1F&, int, bool, bool, dim3, hipStream_t);
extern template void launch_m1_np<float, 32>(const M1F&, int, bool, bool, dim3, hipStream_t);
extern template void launch_m1_np<float, 64>(const M1F&, int, bool, bool, dim3, hipStream_t);
extern template void launch_m1_np<uint16_t, 16>(const M1F&, int, bool, bool, dim3, hipStream_t);
extern template void launch_m1_np<uint16_t, 32>(const M1F&, int, bool, bool, dim3, hipStream_t);
extern template void launch_m1_np<uint16_t, 64>(const M1F&, int, bool, bool, dim3, hipStream_t);
extern template void launch_m1_row_np<float, 16>(const M1F&, bool, bool, dim3, size_t, hipStream_t);
extern template void launch_m1_row_np<float, 32>(const M1F&, bool, bool, dim3, size_t, hipStream_t);
extern template void launch_m1_row_np<float, 64>(const M1F&, bool, bool, dim3, size_t, hipStream_t);
extern template void launch_m1_row_np<uint16_t, 16>(const M1F&, bool, bool, dim3, size_t, hipStream_t);
extern template void launch_m1_row_np<uint16_t, 32>(const M1F&, bool, bool, dim3, size_t, hipStream_t);
extern template void launch_m1_row_np<uint16_t, 64>(const M1F&, bool, bool, dim3, size_t, hipStream_t);

hipError_t launch_m1_fast(const Mamba1Args& a, const Mamba1Plan& plan, const float* ws_h, const float* ws_sdt,
                          hipStream_t s) {
  M1F k{};
  k.x = a.x; k.dt = a.dt; k.dt_bias = a.dt_bias; k.A_log = a.A_log; k.B = a.B; k.C = a.C; k.D = a.D;
  k.z = a.z; k.h0 = a.h0; k.y = a.y; k.h_out = a.h_out; k.states = a.states;
  k.ws_h = ws_h; k.ws_sdt = ws_sdt;
  k.L = a.L; k.Dc = a.Dc; k.per_group = a.Dc / a.G; k.N = (int)a.N; k.G = (int)a.G;
  k.nslices = (int)plan.nslices; k.slice_len = (int)plan.slice_len;
  k.bc_eps = a.bc_eps;
  const int K = (int)plan.lanes_per_channel;
  const bool gate = a.z != nullptr, st = a.states != nullptr;
  const int np = a.N <= 16 ? 16 : a.N <= 32 ? 32 : 64;
  if (K == 16) {  // a 16-lane row per channel, 16 channels per 256-thread block
    const int64_t nb = ((a.Dc + 15) / 16) * plan.nslices * a.batch;
    const dim3 grid((unsigned)nb);
    const size_t dyn = 0;
    if (a.bf16) {
      if (np == 16) launch_m1_row_np<uint16_t, 16>(k, gate, st, grid, dyn, s);
      else if (np == 32) launch_m1_row_np<uint16_t, 32>(k, gate, st, grid, dyn, s);
      else launch_m1_row_np<uint16_t, 64>(k, gate, st, grid, dyn, s);
    } else {
      if (np == 16) launch_m1_row_np<float, 16>(k, gate, st, grid, dyn, s);
      else if (np == 32) launch_m1_row_np<float, 32>(k, gate, st, grid, dyn, s);
      else launch_m1_row_np<float, 64>(k, gate, st, grid, dyn, s);
    }
    return hipGetLastError();
  }
  if (K == 4 && m1_quad_ok(a.N, a.Dc, a.bf16 ? 2 : 4)) {  // a quad per channel, 64 channels per 256-thread block
    const dim3 grid((unsigned)(((a.Dc + 63) / 64) * plan.nslices * a.batch));
    if (a.bf16) {
      if (np == 16) launch_m1_quad_np<uint16_t, 16>(k, gate, st, grid, s);
      else if (np == 32) launch_m1_quad_np<uint16_t, 32>(k, gate, st, grid, s);
      else launch_m1_quad_np<uint16_t, 64>(k, gate, st, grid, s);
    } else {
      if (np == 16) launch_m1_quad_np<float, 16>(k, gate, st, grid, s);
      else if (np == 32) launch_m1_quad_np<float, 32>(k, gate, st, grid, s);
      else launch_m1_quad_np<float, 64>(k, gate, st, grid, s);
    }
    return hipGetLastError();
  }
  const int64_t cpw = 64 / K;
  const dim3 grid((unsigned)(((a.Dc + cpw - 1) / cpw) * plan.nslices * a.batch));
  if (a.bf16) {
    if (np == 16) launch_m1_np<uint16_t, 16>(k, K, gate, st, grid, s);
    else if (np == 32) launch_m1_np<uint16_t, 32>(k, K, gate, st, grid, s);
    else launch_m1_np<uint16_t, 64>(k, K, gate, st, grid, s);
  } else {
    if (np == 16) launch_m1_np<float, 16>(k, K, gate, st, grid, s);
    else if (np == 32) launch_m1_np<float, 32>(k, K, gate, st, grid, s);
    else launch_m1_np<float, 64>(k, K, gate, st, grid, s);
  }
  return hipGetLastError();
}

}  // namespace sscan
