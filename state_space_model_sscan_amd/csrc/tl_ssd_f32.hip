// tl_ssd_f32.hip -- instantiates the token-loop kernels for one (dtype, mode).
#include "tokenloop_impl.hpp"

namespace sscan {
template void dispatch_scan<float, true>(const TLK&, int64_t, bool, bool, hipStream_t);
template void dispatch_step<float, true>(const TLK&, int64_t, bool, hipStream_t);
template void dispatch_pass1<float, true>(const TLK&, int64_t, hipStream_t);
}  // namespace sscan
