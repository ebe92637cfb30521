// m1f_f32_64.hip -- instantiates the Mamba-1 prompt kernel for f32, up to 64 states.
#include "m1_fast_impl.hpp"

namespace sscan {
template void launch_m1_np<float, 64>(const M1F&, int, bool, bool, dim3, hipStream_t);
}  // namespace sscan
