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

// ---------------------------------------------------------------------------
// tile-token score rows: before the attention launch, the keys each query
// tile's workgroups will max into are set to 0 (below the key of any float)
// and the keys past the tile's last key block to -inf; afterwards the keys are
// decoded back to fp32 in place
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void tile_scores_kernel(float* sc, int ntq, int BQ, int Lq, int Lk, int q_off,
                                                          int64_t sb, int64_t sr, int decode) {
  const int row = blockIdx.x;
  const int b = row / ntq, qt = row - b * ntq;
  // the tile's last query, as an absolute position
  const int last = min(min(qt * BQ + BQ, Lq) - 1 + q_off, Lk - 1);
  const int touched = min((last / 64 + 1) * 64, Lk);
  float* p = sc + (int64_t)b * sb + (int64_t)qt * sr;
  uint32_t* u = (uint32_t*)p;
  if (!decode) {
    for (int j = threadIdx.x; j < Lk; j += 256) u[j] = j < touched ? 0u : 0xff800000u;
  } else {
    for (int j = threadIdx.x; j < touched; j += 256) {
      const uint32_t k = u[j];
      const uint32_t f = (k & 0x80000000u) ? (k & 0x7fffffffu) : ~k;
      u[j] = k == 0u ? 0xff800000u : f;
    }
  }
}

hipError_t launch_tile_scores(float* sc, int B, int ntq, int BQ, int Lq, int Lk, int q_off, int64_t sb, int64_t sr,
                              int decode, hipStream_t s) {
  const int64_t rows = (int64_t)B * ntq;
  if (rows <= 0 || Lk <= 0) return hipSuccess;
  hipLaunchKernelGGL(tile_scores_kernel, dim3((unsigned)rows), dim3(256), 0, s, sc, ntq, BQ, Lq, Lk, q_off, sb, sr,
                     decode);
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
