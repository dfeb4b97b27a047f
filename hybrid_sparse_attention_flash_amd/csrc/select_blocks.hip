// Block-level selection over token-score rows at a token budget (gfx950).
//
// HySparse selects 64-token blocks, HySparse2 single tokens; the pages compare
// the two at the same budget of 1024 global + 128 recent tokens (demingchina
// commentary, section 03; airebao HySparse2 news, token-level selection).  The
// block-level side of that comparison on HySparse2's per-tile token scores:
//   block_max_rows_kernel - M[r, c] = max of the row's scores over block c
//                           (one wave per block; -inf past the row end)
//   (top-k of M per row, the library's top-k kernels)
//   expand_blocks_kernel  - each chosen block c becomes the token positions
//                           [64c, min(cols, 64c + 64)), in block order, so a
//                           row's valid positions come first, ascending, and
//                           -1 fills the rest.
#include "common.h"
#include "kernels.h"

namespace hys {

__global__ __launch_bounds__(256) void block_max_rows_kernel(const float* __restrict__ scores, int64_t rows,
                                                            int64_t cols, int64_t row_stride, int nblk,
                                                            float* __restrict__ out) {
  const int64_t w = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (w >= rows * nblk) return;
  const int64_t r = w / nblk;
  const int c = (int)(w - r * nblk);
  const int64_t j = (int64_t)c * 64 + lane;
  float m = j < cols ? scores[r * row_stride + j] : kNegInf;
  m = wave_max(m);
  if (lane == 0) out[r * nblk + c] = m;
}

__global__ __launch_bounds__(256) void expand_blocks_kernel(const int32_t* __restrict__ blocks, int64_t rows,
                                                           int kb, int64_t cols, int32_t* __restrict__ idx) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;   // one output slot
  const int64_t per = (int64_t)kb * 64;
  if (e >= rows * per) return;
  const int64_t r = e / per;
  const int s = (int)(e - r * per);
  const int c = blocks[r * kb + (s >> 6)];
  const int64_t t = (int64_t)c * 64 + (s & 63);
  idx[e] = (c >= 0 && t < cols) ? (int32_t)t : -1;
}

hipError_t launch_block_max_rows(const float* scores, int64_t rows, int64_t cols, int64_t row_stride, int nblk,
                                 float* out, hipStream_t s) {
  const int64_t waves = rows * nblk;
  if (waves == 0) return hipSuccess;
  hipLaunchKernelGGL(block_max_rows_kernel, dim3((unsigned)((waves + 3) / 4)), dim3(256), 0, s, scores, rows, cols,
                     row_stride, nblk, out);
  return hipGetLastError();
}

hipError_t launch_expand_blocks(const int32_t* blocks, int64_t rows, int kb, int64_t cols, int32_t* idx,
                                hipStream_t s) {
  const int64_t n = rows * kb * 64;
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(expand_blocks_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, blocks, rows, kb,
                     cols, idx);
  return hipGetLastError();
}

}  // namespace hys
