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
//   longer rows: each 32768-column chunk keeps its own top-k (exact superset of
//   the row's top-k), then a second pass selects among the chunk winners.
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
// one 1024-thread workgroup per (row, chunk)
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

// vals: row r, position p at vals[r*row_stride + p] (p < cols)
// cmap: if non-null, the original column of position p is cmap[r*row_stride + p]
//       (positions with cmap == -1 are empty); else the column is chunk_base + p.
// Output for (row, chunk): out_idx[(r*nchunk + chunk)*k ...], out_val likewise (if non-null).
//
// Wave w owns positions [2048 w, 2048 w + 2048) of the chunk; lane L holds, in
// slot v, position 2048 w + 64 v + L, so every load instruction reads 256
// contiguous bytes and position order is (wave, slot, lane) order.
template <int VPT, bool CMAP>
__global__ __launch_bounds__(1024) void topk_block_kernel(const float* __restrict__ vals,
                                                          const int32_t* __restrict__ cmap, int64_t rows,
                                                          int64_t cols, int64_t row_stride, int64_t chunk_cols,
                                                          int nchunk, int k, int32_t* __restrict__ out_idx,
                                                          float* __restrict__ out_val, int32_t* __restrict__ count) {
  static_assert(VPT * 64 * 16 == 32768, "a workgroup covers 32768 positions");
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int64_t r = blockIdx.x / nchunk;
  const int chunk = blockIdx.x % nchunk;
  const int64_t cbase = (int64_t)chunk * chunk_cols;
  const int ccols = (int)min(chunk_cols, cols - cbase);
  const float* vr = vals + r * row_stride + cbase;
  const int32_t* mr = CMAP ? cmap + r * row_stride + cbase : nullptr;
  const int pos0 = wave * (64 * VPT) + lane;           // position of slot 0
  // straight-line loads from clamped positions, masked afterwards
  uint32_t key[VPT];
  int cmv[CMAP ? VPT : 1];      // original columns (cmap) of the positions
#pragma unroll
  for (int v = 0; v < VPT; ++v) {
    const int p = pos0 + 64 * v;
    const int pc = min(p, ccols - 1);
    key[v] = __builtin_bit_cast(uint32_t, vr[pc]);
    if constexpr (CMAP) cmv[v] = mr[pc];
  }
#pragma unroll
  for (int v = 0; v < VPT; ++v) {
    const int p = pos0 + 64 * v;
    bool ok = p < ccols;
    if constexpr (CMAP) ok = ok && cmv[v] >= 0;          // cmap -1: an empty candidate slot
    key[v] = ok ? score_key(__builtin_bit_cast(float, key[v])) : 0u;
  }
  // keys >= t in the chunk: per-lane counts, wave totals by DPP, the 16 wave
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
    // smallest and largest valid key of the chunk
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
  // this wave's first tie rank and first output slot, and the chunk total:
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
  const int64_t ob = (r * nchunk + chunk) * (int64_t)k;
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
    if (tk) {
      // the score back from its (valid, hence nonzero) order key
      const uint32_t kk = key[v];
      const uint32_t bits = (kk & 0x80000000u) ? (kk & 0x7fffffffu) : ~kk;
      if constexpr (CMAP) out_idx[ob + slot] = cmv[v];
      else out_idx[ob + slot] = (int32_t)(cbase + pos0 + 64 * v);
      if (out_val) out_val[ob + slot] = __builtin_bit_cast(float, bits);
    }
  }
  for (int p = total + tid; p < k; p += 1024) {
    out_idx[ob + p] = -1;
    if (out_val) out_val[ob + p] = kNegInf;
  }
  if (count && tid == 0) count[r * nchunk + chunk] = total;
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
constexpr int kTopkVPT = 32;
constexpr int64_t kTopkChunk = 1024 * kTopkVPT;      // columns per workgroup pass
constexpr int kTopkMaxLevels = 8;

// Long rows are reduced level by level: level i cuts its input row into
// 32768-column chunks and keeps each chunk's top-k (an exact superset of the
// row's top-k), so its output row is nchunk_i * k candidates long, at most
// 1/8 of its input for k <= 4096; the last level (<= 32768 columns) writes
// the result.  Candidates stay in ascending column order at every level
// (chunk outputs are ascending and chunks are concatenated in order), so a
// tie still resolves to the lowest column.
struct TopkPlan {
  int nlev = 0;                 // reduction levels before the final one
  int64_t nchunk[kTopkMaxLevels] = {};
  int64_t cols[kTopkMaxLevels + 1] = {};   // input columns of each level
};

static TopkPlan topk_plan(int64_t cols, int k) {
  TopkPlan p;
  int64_t c = cols;
  while (c > kTopkChunk && p.nlev < kTopkMaxLevels) {
    p.cols[p.nlev] = c;
    p.nchunk[p.nlev] = (c + kTopkChunk - 1) / kTopkChunk;
    c = p.nchunk[p.nlev] * (int64_t)k;
    ++p.nlev;
  }
  p.cols[p.nlev] = c;
  return p;
}

// Two candidate buffers, used alternately by the levels: the first holds
// level 0's output (the largest), the second level 1's.
size_t topk_workspace_bytes(int64_t rows, int64_t cols, int k) {
  if (cols <= kTopkChunk) return 0;
  const TopkPlan p = topk_plan(cols, k);
  const size_t per = sizeof(float) + sizeof(int32_t);
  size_t n = (size_t)(rows * p.cols[1]) * per;
  if (p.nlev >= 2) n += (size_t)(rows * p.cols[2]) * per;
  return n;
}

size_t topk_workspace_first_bytes(int64_t rows, int64_t cols, int k) {
  if (cols <= kTopkChunk) return 0;
  const TopkPlan p = topk_plan(cols, k);
  return (size_t)(rows * p.cols[1]) * (sizeof(float) + sizeof(int32_t));
}

// Workgroups of the widest launch (rows x chunks of the input row).
int64_t topk_max_workgroups(int64_t rows, int64_t cols, int k) {
  if (cols <= kTopkChunk) return rows;
  const TopkPlan p = topk_plan(cols, k);
  return rows * p.nchunk[0];
}

int64_t topk_chunk_cols() { return kTopkChunk; }

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
    hipLaunchKernelGGL((topk_block_kernel<kTopkVPT, false>), dim3((unsigned)a.rows), dim3(1024), 0, s, a.scores,
                       (const int32_t*)nullptr, a.rows, a.cols, a.row_stride, kTopkChunk, 1, a.k, a.idx,
                       (float*)nullptr, a.count);
    return hipGetLastError();
  }
  const TopkPlan p = topk_plan(a.cols, a.k);
  if (p.cols[p.nlev] > kTopkChunk) return hipErrorInvalidValue;   // excluded by validation
  // candidate buffers: level i writes buffer i % 2
  float* val[2] = {a.cand_val, a.cand_val2};
  int32_t* col[2] = {a.cand_idx, a.cand_idx2};
  for (int lev = 0; lev < p.nlev; ++lev) {
    const int64_t nch = p.nchunk[lev];
    const int64_t out_cols = nch * (int64_t)a.k;
    int32_t* oi = col[lev & 1];
    float* ov = val[lev & 1];
    if (lev == 0) {
      hipLaunchKernelGGL((topk_block_kernel<kTopkVPT, false>), dim3((unsigned)(a.rows * nch)), dim3(1024), 0, s,
                         a.scores, (const int32_t*)nullptr, a.rows, a.cols, a.row_stride, kTopkChunk, (int)nch, a.k,
                         oi, ov, (int32_t*)nullptr);
    } else {
      const int64_t in_cols = p.cols[lev];
      hipLaunchKernelGGL((topk_block_kernel<kTopkVPT, true>), dim3((unsigned)(a.rows * nch)), dim3(1024), 0, s,
                         (const float*)val[(lev - 1) & 1], (const int32_t*)col[(lev - 1) & 1], a.rows, in_cols,
                         in_cols, kTopkChunk, (int)nch, a.k, oi, ov, (int32_t*)nullptr);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    (void)out_cols;
  }
  const int64_t fc = p.cols[p.nlev];
  hipLaunchKernelGGL((topk_block_kernel<kTopkVPT, true>), dim3((unsigned)a.rows), dim3(1024), 0, s,
                     (const float*)val[(p.nlev - 1) & 1], (const int32_t*)col[(p.nlev - 1) & 1], a.rows, fc, fc,
                     kTopkChunk, 1, a.k, a.idx, (float*)nullptr, a.count);
  return hipGetLastError();
}

}  // namespace hys
