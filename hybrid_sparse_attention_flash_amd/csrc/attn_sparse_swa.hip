// Instantiation of the tiled attention engine for: M_SPARSE_SWA.
#include "attn_engine.h"

namespace hys {
template hipError_t launch_mode<M_SPARSE_SWA>(int, int, int, const AttnArgs&, int, hipStream_t);
}  // namespace hys
