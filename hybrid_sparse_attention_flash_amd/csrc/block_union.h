// Per-workgroup union of selected key blocks (QbitAI HySparse article, method
// section: each sparse layer attends to the key blocks the full layer's scores
// selected for its query; TechWalker HySparse write-up, sparse-layer paragraph:
// the selected blocks are gathered into one contiguous key sequence).
//
// A workgroup serves BQ consecutive queries.  Their selections (topk block
// indices each, -1 or out-of-range entries ignored) are merged into one list
// of distinct blocks in ascending order, and for every listed block a bit mask
// of the queries (bit qi for query q0 + qi) that selected it.  Blocks then
// stream through the attention loop once for the whole workgroup; a row that
// did not select a block gets no probability from it.
#pragma once
#include "common.h"

namespace hys {

// Builds s_ulist[0..n) and s_member[0..n) and returns n (the same value in
// every thread).  Called by all 256 threads of the workgroup; contains
// barriers.  Requires nblk <= 32 * NBWMAX and BQ * topk <= UMAX, BQ <= 64.
template <int UMAX, int NBWMAX>
__device__ __forceinline__ int build_block_union(const int32_t* ib, int64_t idx_sr, int topk, int q0, int BQ,
                                                 int Lq, int nblk, uint32_t* s_bitmap, int* s_wpre, int* s_ulist,
                                                 unsigned long long* s_member, int* s_count) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nbw = (nblk + 31) >> 5;
  for (int w = tid; w < nbw; w += 256) s_bitmap[w] = 0u;
  for (int u = tid; u < UMAX; u += 256) s_member[u] = 0ull;
  __syncthreads();
  const int nent = BQ * topk;
  for (int e = tid; e < nent; e += 256) {
    const int qi = e / topk, s = e - qi * topk;
    const int q = q0 + qi;
    if (q < Lq) {
      const int c = ib[(int64_t)q * idx_sr + s];
      if (c >= 0 && c < nblk) atomicOr(&s_bitmap[c >> 5], 1u << (c & 31));
    }
  }
  __syncthreads();
  // exclusive prefix of the words' popcounts: list position of each word's first block
  if (wave == 0) {
    int carry = 0;
    for (int w0 = 0; w0 < nbw; w0 += 64) {
      const int w = w0 + lane;
      const int cnt = (w < nbw) ? __popc(s_bitmap[w]) : 0;
      int x = cnt;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) { const int y = __shfl_up(x, o); if (lane >= o) x += y; }
      if (w < nbw) s_wpre[w] = carry + x - cnt;
      carry += __shfl(x, 63);
    }
    if (lane == 0) *s_count = carry;
  }
  __syncthreads();
  for (int w = tid; w < nbw; w += 256) {
    uint32_t bits = s_bitmap[w];
    int pos = s_wpre[w];
    while (bits) {
      const int bit = __ffs(bits) - 1;
      bits &= bits - 1;
      s_ulist[pos++] = w * 32 + bit;
    }
  }
  for (int e = tid; e < nent; e += 256) {
    const int qi = e / topk, s = e - qi * topk;
    const int q = q0 + qi;
    if (q < Lq) {
      const int c = ib[(int64_t)q * idx_sr + s];
      if (c >= 0 && c < nblk) {
        const int u = s_wpre[c >> 5] + __popc(s_bitmap[c >> 5] & ((1u << (c & 31)) - 1u));
        atomicOr(&s_member[u], 1ull << qi);
      }
    }
  }
  __syncthreads();
  return *s_count;
}

}  // namespace hys
