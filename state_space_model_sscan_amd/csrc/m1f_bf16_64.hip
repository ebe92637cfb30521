// m1f_bf16_64.hip -- instantiates the Mamba-1 prompt kernel for bf16, up to 64 states.
#include "m1_fast_impl.hpp"

namespace sscan {
template void launch_m1_np<uint16_t, 64>(const M1F&, int, bool, bool, dim3, hipStream_t);
}  // namespace sscan
