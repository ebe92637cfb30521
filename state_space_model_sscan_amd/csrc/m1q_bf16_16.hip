// m1q_bf16_16.hip -- instantiates the quad-lane Mamba-1 prompt kernel for one (dtype, state_dim).
#include "m1_quad_impl.hpp"

namespace sscan {
template void launch_m1_quad_np<uint16_t, 16>(const M1F&, bool, bool, dim3, hipStream_t);
}  // namespace sscan
