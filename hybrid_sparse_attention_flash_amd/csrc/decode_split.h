// The all-compute split kernel of the HySparse2 decode step's full layer
// (fp8 cache, D = 128), taken by launch_decode when the cache's layout suits
// its 16-byte LDS-direct loads.
#pragma once
#include "kernels.h"

namespace hys {

bool decode_split_fp8_supported(int D, const DecArgs& a);
hipError_t launch_decode_split_fp8(const DecArgs& a, hipStream_t s);

}  // namespace hys
