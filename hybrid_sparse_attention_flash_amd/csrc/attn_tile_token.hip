// Instantiation of the tiled attention engine for: M_FULL_TILE.
#include "attn_engine.h"

namespace hys {
template hipError_t launch_mode<M_FULL_TILE>(int, int, int, const AttnArgs&, int, hipStream_t);
}  // namespace hys
