// Exact per-row top-k selection on gfx950.
//
// Order: score descending, then column ascending (the lowest index wins a
// tie); entries that are -inf or NaN are never chosen.  The output row holds
// the chosen columns in ascending order, padded with -1, plus their count.
// (TopK over the full layer's importance scores: QbitAI HySparse article,
// method section; TechWalker HySparse write-up, kernel paragraph.)
//
// Method: each score becomes an order-preserving 32-bit key (0 for -inf/NaN).
// The threshold T = the k-th largest key is found without sorting: the
// one-wave kernel bisects over the 32 key bits, each step counting keys >=
// candidate across the row; the workgroup kernel selects T radix-wise, one
// 8-bit digit per round from the top, from an LDS histogram of the keys that
// match the digits chosen so far.  Keys above T are taken; of the keys equal to T the ones with the
// lowest columns fill the remaining slots.  Each thread owns a contiguous
// segment of columns, so an exclusive scan of per-thread counts places every
// chosen column directly at its ascending position.
//
//   short rows (cols <= 2048): one wave per row, up to 32 keys per lane
//   long rows  (cols <= 32768): one 1024-thread workgroup per row, up to 32 keys per thread
//   longer rows: the radix select runs over the whole row with many
//   workgroups per row (a launch per digit, then a count and a write pass).
#include "common.h"
#include "kernels.h"

namespace hys {

__device__ __forceinline__ uint32_t score_key(float x) {
  // valid iff x > -inf (NaN fails the comparison); valid keys are >= 0x00800000.
  // -0 and +0 are equal scores, so both take +0's key (a tie, broken by column).
  return (x > kNegInf) ? f32_order_key(x == 0.f ? 0.f : x) : 0u;
}

// ---------------------------------------------------------------------------
// one wave per row
// ---------------------------------------------------------------------------
template <int V>
__global__ __launch_bounds__(256) void topk_wave_kernel(const float* __restrict__ scores, int64_t rows, int64_t cols,
                                                        int64_t row_stride, int k, int32_t* __restrict__ idx,
                                                        int32_t* __restrict__ count) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const float* sr = scores + row * row_stride;
  const int seg = (int)((cols + 63) / 64);           // columns per lane (<= V)
  const int c0 = lane * seg;
  // unconditional loads from clamped columns (a branch per load would make every
  // load wait for the previous ones), masked afterwards
  float x[V];
#pragma unroll
  for (int v = 0; v < V; ++v) {
    const int c = min(c0 + v, (int)cols - 1);
    x[v] = sr[c];
  }
  uint32_t key[V];
#pragma unroll
  for (int v = 0; v < V; ++v) key[v] = (v < seg && c0 + v < cols) ? score_key(x[v]) : 0u;
  // keys >= t in the row: per-lane counts, wave total by DPP
  auto count_ge = [&](uint32_t t) {
    int n = 0;
#pragma unroll
    for (int v = 0; v < V; ++v) n += (key[v] >= t) ? 1 : 0;
    return wave_sum_i32(n);
  };
  const int nvalid = count_ge(1u);
  uint32_t T = 1u;
  int need = k;   // number of keys equal to T to take (when nvalid > k)
  if (nvalid > k && k > 0) {
    uint32_t t = 0u;
    for (int bit = 31; bit >= 0; --bit) {
      const uint32_t cand = t | (1u << bit);
      if (count_ge(cand) >= k) t = cand;
    }
    T = t;
    need = k - count_ge(T + 1u);
  } else {
    need = 0x7fffffff;
  }
  const bool all = !(nvalid > k && k > 0);
  // ties at T in column order
  int nt = 0;
  if (!all) {
#pragma unroll
    for (int v = 0; v < V; ++v) nt += (key[v] == T) ? 1 : 0;
  }
  int tpre = nt;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) { const int y = __shfl_up(tpre, o); if (lane >= o) tpre += y; }
  tpre -= nt;
  // flags and placement
  int cnt = 0;
  uint32_t take = 0u;
  {
    int tr = tpre;
#pragma unroll
    for (int v = 0; v < V; ++v) {
      bool f;
      if (k <= 0) f = false;
      else if (all) f = key[v] != 0u;
      else if (key[v] > T) f = true;
      else if (key[v] == T) { f = tr < need; ++tr; }
      else f = false;
      if (f) { take |= 1u << v; ++cnt; }
    }
  }
  int pre = cnt;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) { const int y = __shfl_up(pre, o); if (lane >= o) pre += y; }
  const int total = __shfl(pre, 63);
  pre -= cnt;
  int32_t* out = idx + row * (int64_t)k;
#pragma unroll
  for (int v = 0; v < V; ++v)
    if (take & (1u << v)) out[pre++] = c0 + v;
  for (int p = total + lane; p < k; p += 64) out[p] = -1;
  if (count && lane == 0) count[row] = total;
}

// ---------------------------------------------------------------------------
// one 1024-thread workgroup per row (cols <= 32768)
// ---------------------------------------------------------------------------
__device__ __forceinline__ int block_sum_1024(int v, int* sh) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  __syncthreads();
  if (lane == 0) sh[w] = v;
  __syncthreads();
  int t = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) t += sh[i];
  return t;
}

// Row r (one workgroup) is scores[r*row_stride + c], c < cols <= 32768.
// Wave w owns columns [2048 w, 2048 w + 2048); lane L holds, in slot v,
// column 2048 w + 64 v + L, so every load instruction reads 256 contiguous
// bytes and column order is (wave, slot, lane) order.
template <int VPT>
__global__ __launch_bounds__(1024) void topk_block_kernel(const float* __restrict__ vals, int64_t rows, int64_t cols,
                                                          int64_t row_stride, int k, int32_t* __restrict__ out_idx,
                                                          int32_t* __restrict__ count) {
  static_assert(VPT * 64 * 16 == 32768, "a workgroup covers 32768 columns");
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int64_t r = blockIdx.x;
  const int ccols = (int)cols;
  const float* vr = vals + r * row_stride;
  const int pos0 = wave * (64 * VPT) + lane;           // column of slot 0
  // straight-line loads from clamped columns, masked afterwards
  uint32_t key[VPT];
#pragma unroll
  for (int v = 0; v < VPT; ++v) {
    const int p = pos0 + 64 * v;
    key[v] = __builtin_bit_cast(uint32_t, vr[min(p, ccols - 1)]);
  }
#pragma unroll
  for (int v = 0; v < VPT; ++v) {
    const int p = pos0 + 64 * v;
    key[v] = p < ccols ? score_key(__builtin_bit_cast(float, key[v])) : 0u;
  }
  // keys >= t in the row: per-lane counts, wave totals by DPP, the 16 wave
  // totals through LDS
  __shared__ int shc[16];
  auto count_ge = [&](uint32_t t) {
    int n = 0;
#pragma unroll
    for (int v = 0; v < VPT; ++v) n += (key[v] >= t) ? 1 : 0;
    n = wave_sum_i32(n);
    if (lane == 0) shc[wave] = n;
    __syncthreads();
    int tot = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) tot += shc[i];
    __syncthreads();
    return tot;
  };
  const int nvalid = count_ge(1u);
  const bool all = !(nvalid > k && k > 0);
  // ---- the k-th largest key T by radix selection.  The digits start below
  // the leading bits that every valid key shares (those of the smallest and
  // largest valid key): scores of one row mostly share sign and exponent, and
  // a first digit taken from those bits would send nearly every key's atomic
  // to one histogram bin, whose updates serialise.  Each round histograms
  // the next (up to) 8-bit digit of the keys that match the digits chosen so
  // far and picks, scanning digits downward, the one whose bin holds the
  // remaining rank.  need = how many keys equal to T are taken (the rest of k
  // after all keys > T).
  __shared__ __attribute__((aligned(16))) int histc[256 * 32];
  __shared__ int s_pick[2];
  __shared__ uint32_t s_mm[2][16];
  uint32_t T = 0u;
  int need = 0;
  if (!all) {
    // smallest and largest valid key of the row
    uint32_t lo = 0xffffffffu, hi = 0u;
#pragma unroll
    for (int v = 0; v < VPT; ++v) {
      if (key[v] != 0u) { lo = min(lo, key[v]); hi = max(hi, key[v]); }
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      lo = min(lo, (uint32_t)__shfl_xor((int)lo, o));
      hi = max(hi, (uint32_t)__shfl_xor((int)hi, o));
    }
    if (lane == 0) { s_mm[0][wave] = lo; s_mm[1][wave] = hi; }
    __syncthreads();
    lo = 0xffffffffu; hi = 0u;
#pragma unroll
    for (int i = 0; i < 16; ++i) { lo = min(lo, s_mm[0][i]); hi = max(hi, s_mm[1][i]); }
    // bits [31, 32 - common] are shared by every valid key
    const int common = (lo == hi) ? 32 : __clz(lo ^ hi);
    uint32_t prefix = common == 0 ? 0u : (lo & (0xffffffffu << (32 - common)));
    uint32_t pmask = common == 0 ? 0u : (0xffffffffu << (32 - common));
    int krem = k;
    for (int rem_bits = 32 - common; rem_bits > 0;) {
      const int width = rem_bits < 8 ? rem_bits : 8;
      const int shift = rem_bits - width;
      const uint32_t dmask = (1u << width) - 1u;
#pragma unroll
      for (int i = 0; i < 8; ++i) histc[tid + 1024 * i] = 0;
      __syncthreads();
      // 32 copies of each bin, lane l adding to copy l % 32, so lanes that
      // share a digit do not serialise on one LDS address
#pragma unroll
      for (int v = 0; v < VPT; ++v)
        if (key[v] != 0u && (key[v] & pmask) == prefix)
          atomicAdd(&histc[((key[v] >> shift) & dmask) * 32 + (tid & 31)], 1);
      __syncthreads();
      // thread t < 256 takes digit 255 - t; an inclusive scan over t counts
      // the keys with that digit or a larger one
      int c = 0, incl = 0;
      if (tid < 256) {
        const int4* hc = (const int4*)&histc[(255 - tid) * 32];
#pragma unroll
        for (int i = 0; i < 8; ++i) { const int4 x = hc[i]; c += x.x + x.y + x.z + x.w; }
        incl = wave_incl_scan_i32(c);
        if (lane == 63) shc[wave] = incl;
      }
      __syncthreads();
      if (tid < 256) {
        for (int i = 0; i < wave; ++i) incl += shc[i];
        if (incl - c < krem && krem <= incl) { s_pick[0] = 255 - tid; s_pick[1] = incl - c; }
      }
      __syncthreads();
      prefix |= (uint32_t)s_pick[0] << shift;
      pmask |= dmask << shift;
      krem -= s_pick[1];
      rem_bits -= width;
      __syncthreads();                          // s_pick, shc and histc are rewritten next round
    }
    T = prefix;
    need = krem;
  }
  if (k <= 0) { T = 0xffffffffu; need = 0; }      // nothing is taken
  // ---- compaction in position order.  Taken: keys > T, and the first `need`
  // keys equal to T.  (all: T = 0, need = 0 takes every valid key.)
  __shared__ int s_gt[16], s_eq[16];
  {
    int ngt = 0, neq = 0;
#pragma unroll
    for (int v = 0; v < VPT; ++v) { ngt += key[v] > T ? 1 : 0; neq += key[v] == T ? 1 : 0; }
    ngt = wave_sum_i32(ngt);
    neq = wave_sum_i32(neq);
    if (lane == 0) { s_gt[wave] = ngt; s_eq[wave] = neq; }
  }
  __syncthreads();
  // this wave's first tie rank and first output slot, and the row total:
  // wave w takes its keys > T and those of its ties whose rank is below need
  int tie0 = 0, out0 = 0, total = 0;
  {
    int t0 = 0, o0 = 0;
    for (int w = 0; w < 16; ++w) {
      const int eq = s_eq[w];
      if (w == wave) { tie0 = t0; out0 = o0; }
      o0 += s_gt[w] + min(max(need - t0, 0), eq);
      t0 += eq;
    }
    total = o0;
  }
  const int64_t ob = r * (int64_t)k;
  int trun = tie0, orun = out0;
  // tie ranks are needed only in waves that hold keys equal to T (usually one)
  const bool has_eq = __builtin_amdgcn_readfirstlane(s_eq[wave]) != 0;
#pragma unroll
  for (int v = 0; v < VPT; ++v) {
    bool tk = key[v] > T;
    if (has_eq) {
      const bool eq = key[v] == T;
      const unsigned long long be = __ballot(eq);
      const int trank = trun + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(be >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)be, 0u));
      trun += __popcll(be);
      tk = tk || (eq && trank < need);
    }
    const unsigned long long bt = __ballot(tk);
    const int slot = orun + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(bt >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bt, 0u));
    orun += __popcll(bt);
    if (tk) out_idx[ob + slot] = pos0 + 64 * v;
  }
  for (int p = total + tid; p < k; p += 1024) out_idx[ob + p] = -1;
  if (count && tid == 0) count[r] = total;
}

// ---------------------------------------------------------------------------
// int32 fill (used instead of hipMemsetAsync so that captured graphs replay correctly)
__global__ __launch_bounds__(256) void fill_i32_kernel(int32_t* p, int32_t v, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) p[i] = v;
}

hipError_t launch_fill_i32(int32_t* p, int32_t v, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(fill_i32_kernel, dim3((unsigned)blocks), dim3(256), 0, s, p, v, n);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Long rows (cols > 32768): a radix select over the whole row, run by many
// workgroups per row.  The row is cut into chunks (one workgroup each, 8192
// columns per pass over the chunk, chunks of several such pieces when a row
// would otherwise need more than kGridMaxChunks of them).  T is found one digit
// at a time from the top (bits 31..21, 20..10, 9..0 of the order key): every
// workgroup adds its chunk's digit histogram of the keys that match the digits
// chosen so far into the row's global histogram (LDS histogram first, then one
// global atomic per nonzero bin), and the next launch picks the digit whose
// bin holds the remaining rank.  A count pass records each chunk's keys > T
// and keys == T; the write pass turns the preceding chunks' counts into the
// chunk's first output slot and tie rank and places its chosen columns in
// ascending order, exactly as the single-workgroup kernel does inside a chunk.
// Compared with reducing each 32768-column chunk to its own top-k (a candidate
// row of nchunk * k entries that must be reduced again by few workgroups),
// every pass keeps the whole chip busy and no candidate row is built.
// ---------------------------------------------------------------------------
constexpr int kTopkVPT = 32;
constexpr int64_t kTopkChunk = 1024 * kTopkVPT;      // longest row of one workgroup
constexpr int kGridThreads = 256;
constexpr int kGridVPT = 32;
constexpr int kGridPiece = kGridThreads * kGridVPT;  // 8192 columns per pass of a workgroup
constexpr int64_t kGridMaxChunks = 1024;             // chunks per row at most
constexpr int kGridBins1 = 2048, kGridBins2 = 2048, kGridBins3 = 1024;
constexpr int kGridHist = kGridBins1 + kGridBins2 + kGridBins3;   // ints per row
constexpr int kGridState = 8;                        // ints per row

struct GridTopkArgs {
  const float* scores; int64_t rows, cols, row_stride;
  int k;
  int64_t chunk_cols;   // a multiple of kGridPiece
  int nchunk;
  int32_t* hist;        // [rows][kGridHist], zero before the first histogram pass
  int32_t* state;       // [rows][kGridState]: after digit 1 and after digit 2 {mode (1 = take every
                        // valid key), prefix, remaining rank}, then {T, keys == T to take}
  int32_t* counts;      // [rows][nchunk][2]: keys > T, keys == T
  int32_t* idx; int32_t* count;
};

// digit round (0, 1, 2): its lowest key bit, its bin count, its histogram's offset in the row
__device__ __forceinline__ int grid_shift(int round) { return round == 0 ? 21 : (round == 1 ? 10 : 0); }
__device__ __forceinline__ int grid_bins(int round) { return round == 0 ? kGridBins1 : (round == 1 ? kGridBins2 : kGridBins3); }
__device__ __forceinline__ int grid_hist_off(int round) { return round == 0 ? 0 : (round == 1 ? kGridBins1 : kGridBins1 + kGridBins2); }

// Keys of the 8192 columns from col0 on, in the single-workgroup kernel's
// layout: wave w owns columns col0 + [2048 w, 2048 w + 2048), lane L holds
// column col0 + 2048 w + 64 v + L in slot v.  0 for columns past the row's end.
__device__ __forceinline__ void grid_load_keys(const GridTopkArgs& a, int64_t r, int64_t col0, uint32_t (&key)[kGridVPT]) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const float* vr = a.scores + r * a.row_stride;
  const int64_t p0 = col0 + wave * (64 * kGridVPT) + lane;
  const int64_t last = a.cols - 1;
#pragma unroll
  for (int v = 0; v < kGridVPT; ++v) {
    const int64_t c = p0 + 64 * v;
    key[v] = __builtin_bit_cast(uint32_t, vr[c < last ? c : last]);
  }
#pragma unroll
  for (int v = 0; v < kGridVPT; ++v)
    key[v] = (p0 + 64 * v <= last) ? score_key(__builtin_bit_cast(float, key[v])) : 0u;
}

// Sum over the 256 threads (every thread gets it).  sh: 4 ints of LDS.
__device__ __forceinline__ int grid_block_sum(int v, int* sh) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  v = wave_sum_i32(v);
  __syncthreads();
  if (lane == 0) sh[w] = v;
  __syncthreads();
  return sh[0] + sh[1] + sh[2] + sh[3];
}

// Exclusive prefix over the 256 threads in thread order, and the total.
__device__ __forceinline__ int grid_block_excl(int v, int* sh, int& total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int incl = wave_incl_scan_i32(v);
  __syncthreads();
  if (lane == 63) sh[w] = incl;
  __syncthreads();
  int pre = 0;
  for (int i = 0; i < w; ++i) pre += sh[i];
  total = sh[0] + sh[1] + sh[2] + sh[3];
  return pre + incl - v;
}

// The digit of row histogram h (nb bins) that holds rank krem counted from the
// top, and the number of keys in higher bins; total = the histogram's sum.
// Requires krem <= total for a meaningful digit.
__device__ __forceinline__ void grid_pick(const int32_t* h, int nb, int krem, int* sh, int* s_pick, int& digit,
                                          int& above, int& total) {
  const int per = nb / kGridThreads;       // 8 or 4 bins per thread, thread 0 the highest
  const int t = threadIdx.x;
  const int top = nb - per * t;           // this thread's bins are [top - per, top)
  int c = 0;
  for (int i = 0; i < per; ++i) c += h[top - 1 - i];
  const int ex = grid_block_excl(c, sh, total);
  if (ex < krem && krem <= ex + c) {
    int acc = ex;
    for (int i = 0; i < per; ++i) {
      const int hb = h[top - 1 - i];
      if (acc + hb >= krem) { s_pick[0] = top - 1 - i; s_pick[1] = acc; break; }
      acc += hb;
    }
  }
  __syncthreads();
  digit = s_pick[0];
  above = s_pick[1];
  __syncthreads();
}

// Histogram pass of digit ROUND over the keys that match the digits chosen so
// far.  Round 0 also needs no state; rounds 1 and 2 first pick the previous
// digit from the previous histogram (every workgroup of the row does, the
// chunk-0 workgroup records it in the row's state).
template <int ROUND>
__global__ __launch_bounds__(kGridThreads) void topk_grid_hist_kernel(GridTopkArgs a) {
  constexpr int NB = ROUND == 0 ? kGridBins1 : (ROUND == 1 ? kGridBins2 : kGridBins3);
  constexpr int COPIES = ROUND == 0 ? 8 : 1;   // round 0 sees every key: spread each bin over 8 addresses
  constexpr int SHIFT = ROUND == 0 ? 21 : (ROUND == 1 ? 10 : 0);
  __shared__ __attribute__((aligned(16))) int hist[NB * COPIES];
  __shared__ int sh[4], s_pick[2];
  const int tid = threadIdx.x;
  const int64_t r = blockIdx.x / a.nchunk;
  const int chunk = (int)(blockIdx.x % a.nchunk);
  int32_t* hrow = a.hist + r * kGridHist;
  int32_t* st = a.state + r * kGridState;
  uint32_t prefix = 0u, pmask = 0u;
  if constexpr (ROUND > 0) {
    // state after the previous round (round 1: nothing chosen yet, rank k)
    int krem = a.k, mode = 0;
    if constexpr (ROUND == 2) { mode = st[0]; prefix = (uint32_t)st[1]; krem = st[2]; }
    if (mode == 0) {
      int digit, above, total;
      grid_pick(hrow + grid_hist_off(ROUND - 1), grid_bins(ROUND - 1), krem, sh, s_pick, digit, above, total);
      if (ROUND == 1 && total <= a.k) mode = 1;   // no more valid keys than k: every one is taken
      else { prefix |= (uint32_t)digit << grid_shift(ROUND - 1); krem -= above; }
    }
    // this round's slots; the other workgroups of this launch read the previous round's
    if (chunk == 0 && tid == 0) {
      int32_t* o = st + 3 * (ROUND - 1);
      o[0] = mode; o[1] = (int)prefix; o[2] = krem;
    }
    if (mode != 0) return;
    pmask = 0xffffffffu << (SHIFT + (ROUND == 1 ? 11 : 10));
  }
  for (int i = tid; i < NB * COPIES / 4; i += kGridThreads) ((int4*)hist)[i] = make_int4(0, 0, 0, 0);
  __syncthreads();
  const int copy = COPIES > 1 ? (tid & (COPIES - 1)) : 0;
  const int64_t c0 = (int64_t)chunk * a.chunk_cols;
  const int64_t c1 = min(a.cols, c0 + a.chunk_cols);
  // chunk_cols is a multiple of the piece, so a piece never reaches into the
  // next chunk; keys past the row's end are 0
  for (int64_t col0 = c0; col0 < c1; col0 += kGridPiece) {
    uint32_t key[kGridVPT];
    grid_load_keys(a, r, col0, key);
#pragma unroll
    for (int v = 0; v < kGridVPT; ++v)
      if (key[v] != 0u && (key[v] & pmask) == prefix)
        atomicAdd(&hist[((key[v] >> SHIFT) & (NB - 1)) * COPIES + copy], 1);
  }
  __syncthreads();
  int32_t* hg = hrow + grid_hist_off(ROUND);
  for (int b = tid; b < NB; b += kGridThreads) {
    int n = 0;
#pragma unroll
    for (int i = 0; i < COPIES; ++i) n += hist[b * COPIES + i];
    if (n) atomicAdd(&hg[b], n);
  }
}

// Count pass: T = the full key after the last digit, need = the keys equal to
// T to take; each chunk's counts of keys > T and == T.
__global__ __launch_bounds__(kGridThreads) void topk_grid_count_kernel(GridTopkArgs a) {
  __shared__ int sh[4], s_pick[2];
  const int tid = threadIdx.x;
  const int64_t r = blockIdx.x / a.nchunk;
  const int chunk = (int)(blockIdx.x % a.nchunk);
  int32_t* st = a.state + r * kGridState;
  const int mode = st[3];
  uint32_t T = 0u;                               // mode 1: T = 0 and need = 0 take every valid key
  int need = 0;
  if (mode == 0) {
    int digit, above, total;
    const int krem = st[5];
    grid_pick(a.hist + r * kGridHist + grid_hist_off(2), kGridBins3, krem, sh, s_pick, digit, above, total);
    T = (uint32_t)st[4] | (uint32_t)digit;
    need = krem - above;
  }
  if (chunk == 0 && tid == 0) { st[6] = (int)T; st[7] = need; }
  const int64_t c0 = (int64_t)chunk * a.chunk_cols;
  const int64_t c1 = min(a.cols, c0 + a.chunk_cols);
  int ngt = 0, neq = 0;
  for (int64_t col0 = c0; col0 < c1; col0 += kGridPiece) {
    uint32_t key[kGridVPT];
    grid_load_keys(a, r, col0, key);
    // padding keys past the row's end are 0: never > T, and == T only when
    // T = 0, where need = 0
#pragma unroll
    for (int v = 0; v < kGridVPT; ++v) { ngt += key[v] > T ? 1 : 0; neq += key[v] == T ? 1 : 0; }
  }
  ngt = grid_block_sum(ngt, sh);
  neq = grid_block_sum(neq, sh);
  if (tid == 0) {
    int32_t* cn = a.counts + (r * a.nchunk + chunk) * 2;
    cn[0] = ngt;
    cn[1] = neq;
  }
}

// Write pass: chunk j's first output slot is the number of keys taken by
// chunks 0..j-1, its first tie rank the number of keys == T in them.
__global__ __launch_bounds__(kGridThreads) void topk_grid_write_kernel(GridTopkArgs a) {
  __shared__ int sh[4], s_gt[4], s_eq[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t r = blockIdx.x / a.nchunk;
  const int chunk = (int)(blockIdx.x % a.nchunk);
  const int32_t* st = a.state + r * kGridState;
  const uint32_t T = (uint32_t)st[6];
  const int need = st[7];
  const int32_t* cn = a.counts + r * (int64_t)a.nchunk * 2;
  // keys taken by the preceding chunks, 256 chunks at a time
  int orun = 0, trun = 0;
  for (int base = 0; base < chunk; base += kGridThreads) {
    const int i = base + tid;
    const int gt = i < chunk ? cn[2 * i] : 0;
    const int eq = i < chunk ? cn[2 * i + 1] : 0;
    int eqtot;
    const int t0 = trun + grid_block_excl(eq, sh, eqtot);
    const int taken = gt + min(max(need - t0, 0), eq);
    orun += grid_block_sum(taken, sh);
    trun += eqtot;
  }
  int32_t* out = a.idx + r * (int64_t)a.k;
  const int64_t c0 = (int64_t)chunk * a.chunk_cols;
  const int64_t c1 = min(a.cols, c0 + a.chunk_cols);
  for (int64_t col0 = c0; col0 < c1; col0 += kGridPiece) {
    uint32_t key[kGridVPT];
    grid_load_keys(a, r, col0, key);
    const int64_t pw = col0 + wave * (64 * kGridVPT) + lane;   // position of slot 0
    {
      int ngt = 0, neq = 0;
#pragma unroll
      for (int v = 0; v < kGridVPT; ++v) { ngt += key[v] > T ? 1 : 0; neq += key[v] == T ? 1 : 0; }
      ngt = wave_sum_i32(ngt);
      neq = wave_sum_i32(neq);
      __syncthreads();                           // s_gt / s_eq of the previous piece are read
      if (lane == 0) { s_gt[wave] = ngt; s_eq[wave] = neq; }
    }
    __syncthreads();
    // this wave's first tie rank and output slot, and the piece's totals
    int tie0 = trun, out0 = orun, o0 = orun, t0 = trun;
    for (int w = 0; w < 4; ++w) {
      const int eq = s_eq[w];
      if (w == wave) { tie0 = t0; out0 = o0; }
      o0 += s_gt[w] + min(max(need - t0, 0), eq);
      t0 += eq;
    }
    orun = o0;
    trun = t0;
    int tr = tie0, orr = out0;
    const bool has_eq = __builtin_amdgcn_readfirstlane(s_eq[wave]) != 0;
#pragma unroll
    for (int v = 0; v < kGridVPT; ++v) {
      bool tk = key[v] > T;
      if (has_eq) {
        const bool eq = key[v] == T;
        const unsigned long long be = __ballot(eq);
        const int trank = tr + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(be >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)be, 0u));
        tr += __popcll(be);
        tk = tk || (eq && trank < need);
      }
      const unsigned long long bt = __ballot(tk);
      const int slot = orr + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(bt >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bt, 0u));
      orr += __popcll(bt);
      if (tk) out[slot] = (int32_t)(pw + 64 * v);
    }
  }
  if (chunk == a.nchunk - 1) {
    // orun = the row's total (at most k): pad the rest, record the count
    for (int p = orun + tid; p < a.k; p += kGridThreads) out[p] = -1;
    if (a.count && tid == 0) a.count[r] = orun;
  }
}

struct GridPlan { int64_t chunk_cols; int nchunk; };
static GridPlan grid_plan(int64_t cols) {
  const int64_t pieces = (cols + kGridPiece - 1) / kGridPiece;
  const int64_t per = (pieces + kGridMaxChunks - 1) / kGridMaxChunks;      // pieces per chunk
  GridPlan g;
  g.chunk_cols = per * kGridPiece;
  g.nchunk = (int)((cols + g.chunk_cols - 1) / g.chunk_cols);
  return g;
}

size_t topk_workspace_bytes(int64_t rows, int64_t cols, int k) {
  (void)k;
  if (cols <= kTopkChunk) return 0;
  const GridPlan g = grid_plan(cols);
  return (size_t)rows * ((size_t)kGridHist + kGridState + 2 * (size_t)g.nchunk) * sizeof(int32_t);
}

// Workgroups of the widest launch.
int64_t topk_max_workgroups(int64_t rows, int64_t cols, int k) {
  (void)k;
  if (cols <= kTopkChunk) return rows;
  return rows * grid_plan(cols).nchunk;
}

int64_t topk_chunk_cols() { return kTopkChunk; }

int64_t topk_zero_ints(int64_t rows, int64_t cols) { return cols <= kTopkChunk ? 0 : rows * kGridHist; }

hipError_t launch_topk(const TopkArgs& a, hipStream_t s) {
  if (a.rows == 0) return hipSuccess;
  if (a.cols <= 2048 && a.k <= 2048) {
    const unsigned grid = (unsigned)((a.rows + 3) / 4);
    const int64_t seg = (a.cols + 63) / 64;
    if (seg <= 8)
      hipLaunchKernelGGL(topk_wave_kernel<8>, dim3(grid), dim3(256), 0, s, a.scores, a.rows, a.cols, a.row_stride, a.k, a.idx, a.count);
    else
      hipLaunchKernelGGL(topk_wave_kernel<32>, dim3(grid), dim3(256), 0, s, a.scores, a.rows, a.cols, a.row_stride, a.k, a.idx, a.count);
    return hipGetLastError();
  }
  if (a.cols <= kTopkChunk) {
    hipLaunchKernelGGL((topk_block_kernel<kTopkVPT>), dim3((unsigned)a.rows), dim3(1024), 0, s, a.scores, a.rows,
                       a.cols, a.row_stride, a.k, a.idx, a.count);
    return hipGetLastError();
  }
  if (a.k < 1 || !a.ws) return hipErrorInvalidValue;      // k = 0 never reaches here
  const GridPlan g = grid_plan(a.cols);
  GridTopkArgs ga{};
  ga.scores = a.scores; ga.rows = a.rows; ga.cols = a.cols; ga.row_stride = a.row_stride; ga.k = a.k;
  ga.chunk_cols = g.chunk_cols; ga.nchunk = g.nchunk;
  int32_t* w = (int32_t*)a.ws;
  ga.hist = w;
  ga.state = w + a.rows * kGridHist;
  ga.counts = ga.state + a.rows * kGridState;
  ga.idx = a.idx; ga.count = a.count;
  if (!a.hist_zeroed) {
    hipError_t e = launch_fill_i32(ga.hist, 0, a.rows * kGridHist, s);
    if (e != hipSuccess) return e;
  }
  const dim3 grid((unsigned)(a.rows * g.nchunk)), block(kGridThreads);
  hipLaunchKernelGGL(topk_grid_hist_kernel<0>, grid, block, 0, s, ga);
  hipLaunchKernelGGL(topk_grid_hist_kernel<1>, grid, block, 0, s, ga);
  hipLaunchKernelGGL(topk_grid_hist_kernel<2>, grid, block, 0, s, ga);
  hipLaunchKernelGGL(topk_grid_count_kernel, grid, block, 0, s, ga);
  hipLaunchKernelGGL(topk_grid_write_kernel, grid, block, 0, s, ga);
  return hipGetLastError();
}

}  // namespace hys
