// ssd_chunk.hip -- MFMA chunked SSD kernel for gfx950 (placeholder: path disabled).
#include "device_common.hpp"
#include "launch.hpp"

namespace sscan {

bool ssd_chunk_supported(const SSDArgs&) { return false; }
size_t ssd_chunk_ws(const SSDArgs&) { return 0; }
hipError_t launch_ssd_chunk(const SSDArgs&, void*, hipStream_t) { return hipErrorNotSupported; }

}  // namespace sscan
