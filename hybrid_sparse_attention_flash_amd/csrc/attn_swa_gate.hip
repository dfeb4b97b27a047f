// Instantiation of the tiled attention engine for: M_SWA_GATE.
#include "attn_engine.h"

namespace hys {
template hipError_t launch_mode<M_SWA_GATE>(int, int, int, const AttnArgs&, int, hipStream_t);
}  // namespace hys
