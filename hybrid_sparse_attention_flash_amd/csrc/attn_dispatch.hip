// Mode dispatch for the tiled attention engine, and the KV-group score reduction.
#include "common.h"
#include "kernels.h"

namespace hys {

template <int MODE>
hipError_t launch_mode(int qt, int kt, int D, const AttnArgs& a, int grid, hipStream_t s);

// ---------------------------------------------------------------------------
// max over KV-group score slabs
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void reduce_max_kernel(const float* part, int nparts, int64_t stride,
                                                         float* out, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    float m = part[i];
    for (int p = 1; p < nparts; ++p) m = fmaxf(m, part[(int64_t)p * stride + i]);
    out[i] = m;
  }
}

hipError_t launch_reduce_max(const float* part, int nparts, int64_t part_stride, float* out, int64_t n,
                             hipStream_t s) {
  int64_t blocks = (n + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(reduce_max_kernel, dim3((unsigned)blocks), dim3(256), 0, s, part, nparts, part_stride, out, n);
  return hipGetLastError();
}

hipError_t launch_attn(int mode, int qt, int kt, int D, const AttnArgs& a, int grid, hipStream_t s) {
  switch (mode) {
    case M_FULL: return launch_mode<M_FULL>(qt, kt, D, a, grid, s);
    case M_FULL_BLOCK: return launch_mode<M_FULL_BLOCK>(qt, kt, D, a, grid, s);
    case M_FULL_TILE: return launch_mode<M_FULL_TILE>(qt, kt, D, a, grid, s);
    case M_SPARSE_BLOCK: return launch_mode<M_SPARSE_BLOCK>(qt, kt, D, a, grid, s);
    case M_SPARSE_TOKEN: return launch_mode<M_SPARSE_TOKEN>(qt, kt, D, a, grid, s);
    case M_SWA_GATE: return launch_mode<M_SWA_GATE>(qt, kt, D, a, grid, s);
    case M_SPARSE_SWA: return launch_mode<M_SPARSE_SWA>(qt, kt, D, a, grid, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace hys
