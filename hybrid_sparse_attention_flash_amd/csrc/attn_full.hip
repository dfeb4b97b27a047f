// Instantiation of the tiled attention engine for: M_FULL, M_FULL_BLOCK.
#include "attn_engine.h"

namespace hys {
template hipError_t launch_mode<M_FULL>(int, int, int, const AttnArgs&, int, hipStream_t);
template hipError_t launch_mode<M_FULL_BLOCK>(int, int, int, const AttnArgs&, int, hipStream_t);
}  // namespace hys
