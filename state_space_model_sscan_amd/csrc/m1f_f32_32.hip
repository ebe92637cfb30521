// m1f_f32_32.hip -- instantiates the Mamba-1 prompt kernel for f32, up to 32 states.
#include "m1_fast_impl.hpp"

namespace sscan {
template void launch_m1_np<float, 32>(const M1F&, int, bool, bool, dim3, hipStream_t);
}  // namespace sscan
