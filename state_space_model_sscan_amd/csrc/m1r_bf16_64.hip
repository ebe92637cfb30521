// m1r_bf16_64.hip -- instantiates the row-per-channel Mamba-1 prompt kernel for bf16, up to 64 states.
#include "m1_row_impl.hpp"

namespace sscan {
template void launch_m1_row_np<uint16_t, 64>(const M1F&, bool, bool, dim3, size_t, hipStream_t);
}  // namespace sscan
