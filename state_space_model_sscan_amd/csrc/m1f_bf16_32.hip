// m1f_bf16_32.hip -- instantiates the Mamba-1 prompt kernel for bf16, up to 32 states.
#include "m1_fast_impl.hpp"

namespace sscan {
template void launch_m1_np<uint16_t, 32>(const M1F&, int, bool, bool, dim3, hipStream_t);
}  // namespace sscan
