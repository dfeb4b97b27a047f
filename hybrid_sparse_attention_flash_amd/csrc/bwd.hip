// Backward pass of the HySparse hybrid block on gfx950 (v_mfma_f32_16x16x32_bf16
// for dK/dV, v_mfma_f32_32x32x16_bf16 for dQ).
//
// HySparse is trained directly (QbitAI HySparse article, opening summary;
// demingchina HySparse2 commentary, section 06).  With the selection held
// fixed, each attention branch's gradients are those of softmax attention over
// a visible set:
//   P = exp(S - LSE),  dV = P^T dO,  dP = dO V^T,  dS = P (dP - rowsum(dO O)),
//   dQ = scale dS K,   dK = scale dS^T Q,
// summed over the G query heads of a KV head for dK, dV.  Two kernels per
// branch, neither with atomics:
//   bwd_dkdv_causal_kernel - the full layer's dK/dV: 128 keys of one KV head
//     per workgroup, 32 per wave, over the 32-row query blocks that see them.
//   bwd_dkdv_kernel - key-stationary: a workgroup owns 64 keys of one KV head
//     (16 per wave, held in registers as MFMA operands) and walks the query
//     rows that see them (block-sparse: the rows that selected the block) 32
//     at a time for every head of the group, staging Q and dO through LDS both
//     row-major (A operands of S and dP) and transposed (B operands of dK and
//     dV); dK and dV stay in registers and are written once.
//   bwd_dq_kernel - query-stationary: a workgroup owns 128 (query row, head)
//     columns of one KV group (16 rows x 8 heads when the group has 8 or more
//     heads, else 32-row blocks of up to 4 heads) and walks the 64-key tiles
//     they see, staging K (row-major and transposed) and V through LDS once
//     for all of them; dQ stays in registers.
// P and dS come back from the forward's LSE in both kernels.  P and dS leave
// the MFMA in its C layout (lane = one column, rows spread over the 16
// values); they feed the next MFMA as A operands directly, with the other
// operand read in the same permuted row order, so no transpose of P or dS is
// needed.  The block-sparse branch walks per-block lists of the selecting rows
// (dK/dV) and skips key tiles that no row of a 16-row block selected (dQ).

#include <algorithm>

#include "bwd.h"
#include "common.h"
#include "kernels.h"

namespace hys {
namespace {

typedef unsigned int bw_u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int bw_u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ bf16x8 bwf(bw_u32x4 v) { return __builtin_bit_cast(bf16x8, v); }
__device__ __forceinline__ bw_u32x4 cat2(bw_u32x2 lo, bw_u32x2 hi) { return bw_u32x4{lo.x, lo.y, hi.x, hi.y}; }
__device__ __forceinline__ bw_u32x4 zero4() { return bw_u32x4{0u, 0u, 0u, 0u}; }

// eight consecutive values of one 16-byte-aligned chunk packed as MFMA A fragment
__device__ __forceinline__ bw_u32x4 pack8(const float* x) {
  return bw_u32x4{pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]), pack_bf16x2(x[4], x[5]), pack_bf16x2(x[6], x[7])};
}

template <int MODE>
__device__ __forceinline__ bool bw_visible(int i, int j, int L, int Lk, int window, bool bit) {
  bool ok = i < L && j < Lk && j <= i;
  if (MODE == BW_WINDOW) ok = ok && j > i - window;
  if (MODE == BW_BLOCK) ok = ok && bit;
  return ok;
}

// Transposed LDS copy of two rows' 16-byte chunks (8 bf16 each of rows 2rp and
// 2rp+1, columns 8ch..8ch+7): column d receives one dword holding both rows.
// With the lanes of a wave on consecutive row pairs and the row strides
// chosen by the kernels (36, 72 elements), the 64 lanes of each store hit 64
// distinct banks.
template <int TS>
__device__ __forceinline__ void store_t8x2(uint16_t* t, int rp, int ch, bw_u32x4 v0, bw_u32x4 v1) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const uint32_t a = v0[e >> 1], b = v1[e >> 1];
    const uint32_t w = (e & 1) ? ((a >> 16) | (b & 0xffff0000u)) : ((a & 0xffffu) | (b << 16));
    *(uint32_t*)&t[(8 * ch + e) * TS + 2 * rp] = w;
  }
}

// Next row block of a causal dK/dV workgroup: blocks [base, rb_hi) in chunks of 64.
__device__ __forceinline__ bool next_row_block(int lane, int rb_hi, uint64_t& mask, int& base, int& rb) {
  while (mask == 0ull) {
    base += 64;
    if (base >= rb_hi) return false;
    mask = __ballot(base + lane < rb_hi);
  }
  rb = base + __builtin_ctzll(mask);
  mask &= mask - 1ull;
  return true;
}

// dK/dV of the full layer (causal).  A workgroup owns 128 keys of one KV head,
// 32 per wave on v_mfma_f32_32x32x16_bf16, and walks the 32-row query blocks
// from its first key on, once per head of the group, with Q/dO loads issued
// two steps ahead over alternating register sets.  Every staged row serves
// 128 keys here, twice as many as in the 64-key kernel below, which is what
// the dense causal pass needs (its staging, not its latency, is the larger
// cost); row splits are absolute ranges of split_rb 32-row blocks.
template <int MODE, int D>
__global__ __launch_bounds__(256) void bwd_dkdv_causal_kernel(BwdArgs a) {
  constexpr int NC = D / 16;              // 16-wide d chunks of the S and dP contractions
  constexpr int NT = D / 32;              // 32-wide d tiles of dK and dV
  constexpr int RS = D + 8;               // row-major LDS row stride (elements)
  constexpr int TS = 36;                  // transposed LDS row stride: 32 rows + 4
  constexpr int CPR = D / 8;              // 16-byte chunks per row
  constexpr int NIT = 16 * CPR;           // staging items: (row pair, chunk)
  __shared__ __attribute__((aligned(16))) uint16_t s_q[32 * RS];
  __shared__ __attribute__((aligned(16))) uint16_t s_do[32 * RS];
  __shared__ __attribute__((aligned(16))) uint16_t s_qt[D * TS];
  __shared__ __attribute__((aligned(16))) uint16_t s_dot[D * TS];
  __shared__ __attribute__((aligned(16))) float s_lse[32];
  __shared__ __attribute__((aligned(16))) float s_dd[32];
  static_assert(MODE == BW_CAUSAL, "the window and block-sparse branches run bwd_dkdv_kernel");

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ln = lane & 31, hh = lane >> 5;
  // key tiles slowest, so the long causal tiles (small k0) are dispatched first
  // split slowest: the workgroups running together read the same absolute
  // range of query rows, so their Q and dO stay in cache; within a split the
  // key tiles (long causal tiles first) then the (batch, KV head) pairs
  const int nbh = a.Hkv * a.B, ntk = (a.Lk + 127) / 128;
  const int split = blockIdx.x / (ntk * nbh), tile = blockIdx.x - split * (ntk * nbh);
  const int kt = tile / nbh, gb = tile - kt * nbh;
  const int g = gb % a.Hkv, b = gb / a.Hkv;
  const int k0 = kt * 128, kw0 = k0 + 32 * wave;
  const int nrb = (a.L + 31) / 32;

  // this wave's 32 keys and values as B operands: lane (ln, hh) holds key ln, d = 16c + 8hh + [0, 8)
  bw_u32x4 kf[NC], vf[NC];
  {
    const int key = kw0 + ln;
    const bool ok = key < a.Lk;
    const int64_t off = (int64_t)b * a.k_sb + (int64_t)(ok ? key : 0) * a.k_st + (int64_t)g * a.k_sh + 8 * hh;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      kf[c] = ok ? *(const bw_u32x4*)(a.k + off + 16 * c) : zero4();
      vf[c] = ok ? *(const bw_u32x4*)(a.v + off + 16 * c) : zero4();
    }
  }
  f32x16 dk_acc[NT], dv_acc[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int i = 0; i < 16; ++i) { dk_acc[t][i] = 0.f; dv_acc[t][i] = 0.f; }

  int rb_hi = nrb;
  // this workgroup's share of the row blocks that can see the tile: absolute
  // row blocks [split * split_rb, (split + 1) * split_rb)
  const int rb_first = max(k0 / 32, split * a.split_rb);
  rb_hi = min(rb_hi, (split + 1) * a.split_rb);
  uint64_t mask = 0ull;
  int base = rb_first - 64, rb = 0, h = 0;
  bool have = rb_first < rb_hi && next_row_block(lane, rb_hi, mask, base, rb);
  const bool did = have;

  // staging item tid (when tid < NIT): rows 2rp, 2rp+1 of the block, 16-byte chunk ch.
  // Two register sets alternate (the loop is unrolled by two), so the loads of
  // a step are issued two steps before it is staged into LDS.
  const int rp = tid & 15, sch = tid >> 4;
  const bool stager = tid < NIT;
  bw_u32x4 pq[2][2], pdo[2][2];
  float plse[2] = {kNegInf, kNegInf}, pdd[2] = {0.f, 0.f};
  uint32_t pok[2] = {0u, 0u};             // bit u: staging row u in range; 4: lse row
  int srb[2] = {0, 0};
  bool shave[2] = {false, false};
  auto issue = [&](auto set_tag, int rbi, int hq) __attribute__((always_inline)) {
    constexpr int S = decltype(set_tag)::value;
    // every load is issued unconditionally from a clamped, in-bounds address
    // and the out-of-range values are replaced when the set is staged: with
    // no load under a branch and no use before then, the wait before a set is
    // staged covers that set's loads only
    const int r0 = rbi * 32;
    const int ch = stager ? sch : 0;
    uint32_t okm = 0u;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int i = r0 + 2 * rp + u;
      const bool ok = stager && i < a.L;
      const int ii = ok ? i : 0;
      okm |= (ok ? 1u : 0u) << u;
      pq[S][u] = *(const bw_u32x4*)(a.q + (int64_t)b * a.q_sb + (int64_t)ii * a.q_st + (int64_t)hq * a.q_sh + 8 * ch);
      pdo[S][u] = *(const bw_u32x4*)(a.dO + (int64_t)b * a.do_sb + (int64_t)ii * a.do_st + (int64_t)hq * a.do_sh +
                                     8 * ch);
    }
    {
      const int i = r0 + (tid & 31);
      const bool ok = i < a.L;
      okm |= (ok ? 4u : 0u);
      const int64_t o = ((int64_t)b * a.Hq + hq) * a.L + (ok ? i : 0);
      plse[S] = a.lse[o];
      pdd[S] = a.Dd[o];
    }
    pok[S] = okm;
  };
  // the step after the current (row block, head): heads fastest
  auto advance = [&]() __attribute__((always_inline)) {
    if (!have) return;
    if (++h >= a.G) {
      h = 0;
      have = next_row_block(lane, rb_hi, mask, base, rb);
    }
  };
  // take the next step into set S and issue its loads (after finding the
  // step that follows, whose rare bitmap read would otherwise wait for them)
  auto fill = [&](auto set_tag) __attribute__((always_inline)) {
    constexpr int S = decltype(set_tag)::value;
    const int hs = h;
    shave[S] = have;
    srb[S] = rb;
    advance();
    if (shave[S]) issue(set_tag, srb[S], g * a.G + hs);
  };

  auto step = [&](auto set_tag) __attribute__((always_inline)) {
    constexpr int S = decltype(set_tag)::value;
    const int cur_r0 = srb[S] * 32;
    __syncthreads();                      // the previous step's LDS reads are done
    const uint32_t okm = pok[S];
    if (stager) {
      bw_u32x4 xq[2], xd[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const bool ok = (okm >> u) & 1u;
        xq[u] = ok ? pq[S][u] : zero4();
        xd[u] = ok ? pdo[S][u] : zero4();
        *(bw_u32x4*)&s_q[(2 * rp + u) * RS + 8 * sch] = xq[u];
        *(bw_u32x4*)&s_do[(2 * rp + u) * RS + 8 * sch] = xd[u];
      }
      store_t8x2<TS>(s_qt, rp, sch, xq[0], xq[1]);
      store_t8x2<TS>(s_dot, rp, sch, xd[0], xd[1]);
    }
    if (tid < 32) {
      s_lse[tid] = (okm & 4u) ? plse[S] * kLog2e : kNegInf;
      s_dd[tid] = (okm & 4u) ? pdd[S] : 0.f;
    }
    __syncthreads();
    // this set now takes the step two ahead, whose loads overlap two steps of compute
    fill(set_tag);

    bool any = kw0 <= cur_r0 + 31 && kw0 < a.Lk;
    if (any) {
      f32x16 s, dp;
#pragma unroll
      for (int i = 0; i < 16; ++i) { s[i] = 0.f; dp[i] = 0.f; }
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const bw_u32x4 aq = *(const bw_u32x4*)&s_q[ln * RS + 16 * c + 8 * hh];
        const bw_u32x4 ad = *(const bw_u32x4*)&s_do[ln * RS + 16 * c + 8 * hh];
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bwf(aq), bwf(kf[c]), s, 0, 0, 0);
        dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bwf(ad), bwf(vf[c]), dp, 0, 0, 0);
      }
      // element i: query row 8(i/4) + 4hh + i%4 of the block, key kw0 + ln.
      // A block every one of whose rows sees all 32 keys skips the
      // per-element test (wave-uniform: away from the diagonal, the window
      // edges, partly selected blocks and the ragged ends).
      bool full = kw0 + 31 <= cur_r0 && cur_r0 + 31 < a.L && kw0 + 31 < a.Lk;
      float p[16], ds[16];
      const int key = kw0 + ln;
      if (full) {
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          const f32x4 l4 = *(const f32x4*)&s_lse[8 * i4 + 4 * hh];
          const f32x4 d4 = *(const f32x4*)&s_dd[8 * i4 + 4 * hh];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int i = 4 * i4 + e;
            const float pv = __builtin_amdgcn_exp2f(fmaf(s[i], a.scale_log2, -l4[e]));
            p[i] = pv;
            ds[i] = pv * (dp[i] - d4[e]);
          }
        }
      } else {
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          const f32x4 l4 = *(const f32x4*)&s_lse[8 * i4 + 4 * hh];
          const f32x4 d4 = *(const f32x4*)&s_dd[8 * i4 + 4 * hh];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int i = 4 * i4 + e, row = 8 * i4 + 4 * hh + e;
            const bool vis = bw_visible<MODE>(cur_r0 + row, key, a.L, a.Lk, a.window, true) && l4[e] != kNegInf;
            const float pv = vis ? __builtin_amdgcn_exp2f(fmaf(s[i], a.scale_log2, -l4[e])) : 0.f;
            p[i] = pv;
            ds[i] = pv * (dp[i] - d4[e]);
          }
        }
      }
      // A fragments: k-slot 8hh + j of chunk kc is row 16kc + 8(j/4) + 4hh + j%4, i.e. value 8kc + j
      const bw_u32x4 pa0 = pack8(p), pa1 = pack8(p + 8);
      const bw_u32x4 da0 = pack8(ds), da1 = pack8(ds + 8);
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const uint16_t* td = &s_dot[(32 * t + ln) * TS + 4 * hh];
        const uint16_t* tq = &s_qt[(32 * t + ln) * TS + 4 * hh];
        const bw_u32x4 bd0 = cat2(*(const bw_u32x2*)(td), *(const bw_u32x2*)(td + 8));
        const bw_u32x4 bd1 = cat2(*(const bw_u32x2*)(td + 16), *(const bw_u32x2*)(td + 24));
        const bw_u32x4 bq0 = cat2(*(const bw_u32x2*)(tq), *(const bw_u32x2*)(tq + 8));
        const bw_u32x4 bq1 = cat2(*(const bw_u32x2*)(tq + 16), *(const bw_u32x2*)(tq + 24));
        dv_acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bwf(pa0), bwf(bd0), dv_acc[t], 0, 0, 0);
        dv_acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bwf(pa1), bwf(bd1), dv_acc[t], 0, 0, 0);
        dk_acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bwf(da0), bwf(bq0), dk_acc[t], 0, 0, 0);
        dk_acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bwf(da1), bwf(bq1), dk_acc[t], 0, 0, 0);
      }
    }
  };

  fill(std::integral_constant<int, 0>{});
  fill(std::integral_constant<int, 1>{});
  while (shave[0]) {
    step(std::integral_constant<int, 0>{});
    if (!shave[1]) break;
    step(std::integral_constant<int, 1>{});
  }

  // dK, dV in C layout: lane (ln, hh) holds d = 32t + ln of keys kw0 + 8(i/4) + 4hh + i%4
  if (a.nsplit > 1) {
    if (tid == 0) a.flags[blockIdx.x] = did ? 1 : 0;
    if (!did) return;
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = kw0 + 8 * (i >> 2) + 4 * hh + (i & 3);
        if (key >= a.Lk) continue;
        const int64_t o = ((((int64_t)split * a.B + b) * a.Lk + key) * a.Hkv + g) * D + 32 * t + ln;
        a.part_k[o] = dk_acc[t][i] * a.scale;
        a.part_v[o] = dv_acc[t][i];
      }
    return;
  }
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int key = kw0 + 8 * (i >> 2) + 4 * hh + (i & 3);
      if (key >= a.Lk) continue;
      const int64_t o = (int64_t)b * a.dk_sb + (int64_t)key * a.dk_st + (int64_t)g * a.dk_sh + 32 * t + ln;
      const float kv = dk_acc[t][i] * a.scale, vv = dv_acc[t][i];
      if (a.acc_kv) { a.dk[o] += kv; a.dv[o] += vv; }
      else { a.dk[o] = kv; a.dv[o] = vv; }
    }
}

// dK/dV, key-stationary.  A workgroup owns one 64-key block of one KV head and
// walks the query rows that see the block, 32 per step, once per head of the
// group (heads fastest): in block mode the list of rows that selected the block
// (ascending, built by bwd_rowlist_kernel), in the causal and window modes the
// rows from the block's first key on (to the last row whose window reaches it).  Wave w holds keys 16w .. 16w + 15 of the block as B
// operands of v_mfma_f32_16x16x32_bf16, so K/V fragments and dK/dV take half
// the registers of the causal kernel's 32-key waves and two workgroups fit on
// a CU (two waves per SIMD, each hiding the other's LDS, MFMA and barrier
// latency).  Every row of a block-mode step selected the block, so only
// causality (and the window) and the rows' end are tested per element.  The
// list goes through an LDS window, so a step's Q/dO loads, issued one step
// ahead, take their rows from LDS and never wait on a global index load.  Row
// splits cut a block's rows into ranges of split_rb * 32, one workgroup each;
// each writes flagged partial sums that bwd_kv_reduce_kernel adds in split
// order.
//
// 16x16x32 lane layout (lane l, li = l % 16, lg = l / 16): A[m = li][k = 8lg + j],
// B[k = 8lg + j][n = li], C[m = 4lg + i][n = li].  S = Q K^T and dP = dO V^T
// come out as C[row][key] in two 16-row blocks, so lane (li, lg) holds key li
// for rows 4lg + i and 16 + 4lg + i: those eight values are the lane's A
// fragment of P^T (dV = P^T dO) and dS^T (dK = dS^T Q) with k-slot j standing
// for row 4lg + j % 4 + 16 (j / 4), and the B operands (dO, Q) are read from
// the transposed LDS copies in that row order.
template <int MODE, int D>
__global__ __launch_bounds__(256, 2) void bwd_dkdv_kernel(BwdArgs a) {
  constexpr int NK = D / 32;              // 32-wide k-steps of S and dP
  constexpr int NDB = D / 16;             // 16-wide d blocks of dK and dV
  constexpr int RS = D + 8;               // row-major LDS row stride (elements)
  constexpr int TS = 36;                  // transposed LDS row stride: 32 rows + 4
  constexpr int CPR = D / 8;              // 16-byte chunks per row
  constexpr int NIT = 16 * CPR;           // staging items: (row pair, chunk)
  constexpr int NL = MODE == BW_BLOCK ? 2048 : 1;   // list window (entries)
  __shared__ __attribute__((aligned(16))) uint16_t s_q[32 * RS];
  __shared__ __attribute__((aligned(16))) uint16_t s_do[32 * RS];
  __shared__ __attribute__((aligned(16))) uint16_t s_qt[D * TS];
  __shared__ __attribute__((aligned(16))) uint16_t s_dot[D * TS];
  __shared__ __attribute__((aligned(16))) float s_lse[32];
  __shared__ __attribute__((aligned(16))) float s_dd[32];
  __shared__ __attribute__((aligned(16))) int s_row[32];
  __shared__ int s_list[NL];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int li = lane & 15, lg = lane >> 4;
  // blocks slowest within a split, split slowest: the long causal blocks
  // (small kb) are dispatched first
  const int nbh = a.Hkv * a.B, nkb = (a.Lk + 63) / 64;
  const int split = blockIdx.x / (nkb * nbh), tile = blockIdx.x - split * (nkb * nbh);
  const int kb = tile / nbh, gb = tile - kb * nbh;
  const int g = gb % a.Hkv, b = gb / a.Hkv;
  const int kw0 = kb * 64 + 16 * wave;
  const int gs = a.ng > 1 ? g : 0;

  // B operands of S (K^T) and dP (V^T): lane (li, lg) holds key kw0 + li, d = 32c + 8lg + [0, 8)
  bw_u32x4 kf[NK], vf[NK];
  {
    const int key = kw0 + li;
    const bool ok = key < a.Lk;
    const int64_t off = (int64_t)b * a.k_sb + (int64_t)(ok ? key : 0) * a.k_st + (int64_t)g * a.k_sh + 8 * lg;
#pragma unroll
    for (int c = 0; c < NK; ++c) {
      kf[c] = ok ? *(const bw_u32x4*)(a.k + off + 32 * c) : zero4();
      vf[c] = ok ? *(const bw_u32x4*)(a.v + off + 32 * c) : zero4();
    }
  }
  f32x4 dk_acc[NDB], dv_acc[NDB];
#pragma unroll
  for (int t = 0; t < NDB; ++t) { dk_acc[t] = f32x4{0.f, 0.f, 0.f, 0.f}; dv_acc[t] = f32x4{0.f, 0.f, 0.f, 0.f}; }

  // the block's rows and this workgroup's share of them: entries [p_first, p_hi)
  // (causal and window: entry p is row 64kb + p)
  const int row0 = kb * 64;
  int rcnt;
  const int32_t* rlist = nullptr;
  if constexpr (MODE == BW_BLOCK) {
    const int64_t tl = (int64_t)(gs * a.B + b) * nkb + kb;
    rlist = a.rowlist + tl * a.L;
    rcnt = __builtin_amdgcn_readfirstlane(a.rowcnt[tl]);
  } else if constexpr (MODE == BW_WINDOW) {
    rcnt = max(0, min(a.L - row0, 64 + a.window - 1));
  } else {
    rcnt = max(0, a.L - row0);
  }
  const int p_first = split * a.split_rb * 32;
  const int p_hi = min(rcnt, p_first + a.split_rb * 32);
  const bool did = p_first < p_hi;
  int pos = p_first, h = 0;               // the next step to issue
  bool have = did;
  int win0 = -(NL + 32);                  // no window loaded yet
  // list entries [p0, p0 + NL) into s_list; every thread calls it, and no read
  // of the old window is pending (the issue reads it synchronously)
  auto load_window = [&](int p0) __attribute__((always_inline)) {
    __syncthreads();
    for (int e = tid; e < NL; e += 256) {
      const int p = p0 + e;
      s_list[e] = p < p_hi ? rlist[p] : 0;
    }
    __syncthreads();
    win0 = p0;
  };

  // the step in flight: staging item tid (when tid < NIT) holds rows 2rp,
  // 2rp + 1 of the step, 16-byte chunk ch; thread tid < 32 the LSE and
  // rowsum(dO O) of entry tid.  Every load is issued unconditionally from a
  // clamped address.
  const int rp = tid & 15, sch = tid >> 4;
  const bool stager = tid < NIT;
  bw_u32x4 pq[2], pdo[2];
  float plse = kNegInf, pdd = 0.f;
  int prow = 0;
  uint32_t pok = 0u;                      // bit u: staging row u in range; 4: lse row
  auto issue = [&](int p0, int hq) __attribute__((always_inline)) {
    const int lw = p0 - win0;             // the step's first entry in the window
    const int ch = stager ? sch : 0;
    uint32_t okm = 0u;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const bool ok = stager && p0 + 2 * rp + u < p_hi;
      const int i = MODE == BW_BLOCK ? s_list[lw + 2 * rp + u] : row0 + p0 + 2 * rp + u;
      const int ii = ok ? i : 0;
      okm |= (ok ? 1u : 0u) << u;
      pq[u] = *(const bw_u32x4*)(a.q + (int64_t)b * a.q_sb + (int64_t)ii * a.q_st + (int64_t)hq * a.q_sh + 8 * ch);
      pdo[u] = *(const bw_u32x4*)(a.dO + (int64_t)b * a.do_sb + (int64_t)ii * a.do_st + (int64_t)hq * a.do_sh + 8 * ch);
    }
    if (tid < 32) {
      const bool ok = p0 + tid < p_hi;
      const int i = MODE == BW_BLOCK ? s_list[lw + tid] : row0 + p0 + tid;
      okm |= ok ? 4u : 0u;
      prow = ok ? i : a.L;
      const int64_t o = ((int64_t)b * a.Hq + hq) * a.L + (ok ? i : 0);
      plse = a.lse[o];
      pdd = a.Dd[o];
    }
    pok = okm;
  };
  // issue the next step (loading the window first when the step leaves it)
  auto issue_next = [&]() __attribute__((always_inline)) {
    if constexpr (MODE == BW_BLOCK)
      if (pos + 32 > win0 + NL) load_window(pos);
    issue(pos, g * a.G + h);
    if (++h >= a.G) { h = 0; pos += 32; have = pos < p_hi; }
  };

  int cur_pos = pos;
  if (have) issue_next();
  while (did) {
    const int step_pos = cur_pos;
    const bool last = !have;
    __syncthreads();                      // the previous step's LDS reads are done
    if (stager) {
      bw_u32x4 xq[2], xd[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const bool ok = (pok >> u) & 1u;
        xq[u] = ok ? pq[u] : zero4();
        xd[u] = ok ? pdo[u] : zero4();
        *(bw_u32x4*)&s_q[(2 * rp + u) * RS + 8 * sch] = xq[u];
        *(bw_u32x4*)&s_do[(2 * rp + u) * RS + 8 * sch] = xd[u];
      }
      store_t8x2<TS>(s_qt, rp, sch, xq[0], xq[1]);
      store_t8x2<TS>(s_dot, rp, sch, xd[0], xd[1]);
    }
    if (tid < 32) {
      s_lse[tid] = (pok & 4u) ? plse * kLog2e : kNegInf;
      s_dd[tid] = (pok & 4u) ? pdd : 0.f;
      s_row[tid] = prow;
    }
    __syncthreads();
    // the next step's loads overlap this step's compute
    cur_pos = pos;
    if (have) issue_next();

    // the step's rows: entries step_pos .. step_pos + nval - 1, ascending
    const int nval = min(32, p_hi - step_pos);
    const int r_first = s_row[0];
    const int r_last = s_row[nval - 1];
    bool any = kw0 <= r_last && kw0 < a.Lk;
    if (MODE == BW_WINDOW) any = any && r_first - a.window < kw0 + 15;
    if (any) {
      f32x4 s[2], dp[2];
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        s[rb] = f32x4{0.f, 0.f, 0.f, 0.f};
        dp[rb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < NK; ++c) {
          const bw_u32x4 aq = *(const bw_u32x4*)&s_q[(16 * rb + li) * RS + 32 * c + 8 * lg];
          const bw_u32x4 ad = *(const bw_u32x4*)&s_do[(16 * rb + li) * RS + 32 * c + 8 * lg];
          s[rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bwf(aq), bwf(kf[c]), s[rb], 0, 0, 0);
          dp[rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bwf(ad), bwf(vf[c]), dp[rb], 0, 0, 0);
        }
      }
      // element (rb, i): row 16rb + 4lg + i of the step, key kw0 + li; a step
      // whose 32 rows all lie at or past the wave's last key skips the test
      bool full = nval == 32 && kw0 + 15 <= r_first && kw0 + 15 < a.Lk;
      if (MODE == BW_WINDOW) full = full && r_last - a.window < kw0;
      const int key = kw0 + li;
      float p[8], ds[8];
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        const int r0 = 16 * rb + 4 * lg;
        const f32x4 l4 = *(const f32x4*)&s_lse[r0];
        const f32x4 d4 = *(const f32x4*)&s_dd[r0];
        const int4 q4 = *(const int4*)&s_row[r0];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int qrow = e == 0 ? q4.x : e == 1 ? q4.y : e == 2 ? q4.z : q4.w;
          // entries past the list's end carry row L and LSE -inf
          bool vis = qrow < a.L && key <= qrow && key < a.Lk && l4[e] != kNegInf;
          if (MODE == BW_WINDOW) vis = vis && key > qrow - a.window;
          vis = vis || full;
          const float pv = vis ? __builtin_amdgcn_exp2f(fmaf(s[rb][e], a.scale_log2, -l4[e])) : 0.f;
          p[4 * rb + e] = pv;
          ds[4 * rb + e] = pv * (dp[rb][e] - d4[e]);
        }
      }
      // A fragments of P^T and dS^T: k-slot j is row 4lg + j % 4 + 16 (j / 4)
      const bw_u32x4 pa = pack8(p), da = pack8(ds);
#pragma unroll
      for (int t = 0; t < NDB; ++t) {
        // B fragments: d = 16t + li, rows 4lg .. 4lg + 3 and 16 + 4lg .. 16 + 4lg + 3
        const uint16_t* td = &s_dot[(16 * t + li) * TS + 4 * lg];
        const uint16_t* tq = &s_qt[(16 * t + li) * TS + 4 * lg];
        const bw_u32x4 bd = cat2(*(const bw_u32x2*)(td), *(const bw_u32x2*)(td + 16));
        const bw_u32x4 bq = cat2(*(const bw_u32x2*)(tq), *(const bw_u32x2*)(tq + 16));
        dv_acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bwf(pa), bwf(bd), dv_acc[t], 0, 0, 0);
        dk_acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bwf(da), bwf(bq), dk_acc[t], 0, 0, 0);
      }
    }
    if (last) break;
  }

  // dK, dV in C layout: lane (li, lg) holds d = 16t + li of keys kw0 + 4lg + i
  if (a.nsplit > 1) {
    if (tid == 0) a.flags[blockIdx.x] = did ? 1 : 0;
    if (!did) return;
#pragma unroll
    for (int t = 0; t < NDB; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = kw0 + 4 * lg + i;
        if (key >= a.Lk) continue;
        const int64_t o = ((((int64_t)split * a.B + b) * a.Lk + key) * a.Hkv + g) * D + 16 * t + li;
        a.part_k[o] = dk_acc[t][i] * a.scale;
        a.part_v[o] = dv_acc[t][i];
      }
    return;
  }
#pragma unroll
  for (int t = 0; t < NDB; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int key = kw0 + 4 * lg + i;
      if (key >= a.Lk) continue;
      const int64_t o = (int64_t)b * a.dk_sb + (int64_t)key * a.dk_st + (int64_t)g * a.dk_sh + 16 * t + li;
      const float kv = dk_acc[t][i] * a.scale, vv = dv_acc[t][i];
      if (a.acc_kv) { a.dk[o] += kv; a.dv[o] += vv; }
      else { a.dk[o] = kv; a.dv[o] = vv; }
    }
}

// dk, dv (+)= the flagged partial sums of the row splits, in split order (one
// flag per dK/dV workgroup of tw keys: 128 causal, 64 window and block-sparse)
__global__ __launch_bounds__(256) void bwd_kv_reduce_kernel(BwdArgs a, int D, int tw) {
  const int n4 = D / 4;
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t n = (int64_t)a.B * a.Lk * a.Hkv * n4;
  if (e >= n) return;
  const int d4 = (int)(e % n4);
  int64_t t = e / n4;
  const int g = (int)(t % a.Hkv);
  t /= a.Hkv;
  const int key = (int)(t % a.Lk), b = (int)(t / a.Lk);
  const int nbh = a.Hkv * a.B, ntk = (a.Lk + tw - 1) / tw;
  const int64_t f0 = (int64_t)(key / tw) * nbh + (int64_t)b * a.Hkv + g;      // split s at f0 + s * ntk * nbh
  const int64_t o = (int64_t)b * a.dk_sb + (int64_t)key * a.dk_st + (int64_t)g * a.dk_sh + 4 * d4;
  f32x4 sk = {0.f, 0.f, 0.f, 0.f}, sv = {0.f, 0.f, 0.f, 0.f};
  if (a.acc_kv) {
    sk = *(const f32x4*)(a.dk + o);
    sv = *(const f32x4*)(a.dv + o);
  }
  for (int s = 0; s < a.nsplit; ++s) {
    if (!a.flags[f0 + (int64_t)s * ntk * nbh]) continue;
    const int64_t po = ((((int64_t)s * a.B + b) * a.Lk + key) * a.Hkv + g) * D + 4 * d4;
    sk += *(const f32x4*)(a.part_k + po);
    sv += *(const f32x4*)(a.part_v + po);
  }
  *(f32x4*)(a.dk + o) = sk;
  *(f32x4*)(a.dv + o) = sv;
}

// Next 64-key tile of a dQ workgroup (block mode: the union of its rows'
// selections, from the 16-row union bitmaps of its row blocks rb0 .. rb0+nrbw-1).
template <int MODE>
__device__ __forceinline__ bool next_key_tile(const BwdArgs& a, int gs, int b, int nrb16, int rb0, int nrbw, int c_hi,
                                              uint32_t& bits, int& wi, int& c) {
  if (MODE != BW_BLOCK) { ++c; return c <= c_hi; }
  while (bits == 0u) {
    ++wi;
    if (wi * 32 > c_hi) return false;
    uint32_t u = 0u;
    for (int r = 0; r < nrbw; ++r) u |= a.tilebits16[((int64_t)(gs * a.B + b) * nrb16 + rb0 + r) * a.nwords + wi];
    const int n = c_hi - wi * 32;
    if (n < 31) u &= (2u << n) - 1u;
    bits = u;
  }
  c = wi * 32 + __builtin_ctz(bits);
  bits &= bits - 1u;
  return true;
}

template <int MODE, int D>
__global__ __launch_bounds__(256) void bwd_dq_kernel(BwdArgs a) {
  constexpr int NC = D / 16;
  constexpr int NT = D / 32;
  constexpr int RS = D + 8;               // row-major K, V row stride
  constexpr int TS = 72;                  // transposed K row stride: 64 keys + 8
  constexpr int CPR = D / 8;
  constexpr int NPASS = 32 * CPR / 256;   // staging items (key pair, chunk) per thread
  __shared__ __attribute__((aligned(16))) uint16_t s_k[64 * RS];
  __shared__ __attribute__((aligned(16))) uint16_t s_v[64 * RS];
  __shared__ __attribute__((aligned(16))) uint16_t s_kt[D * TS];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ln = lane & 31, hh = lane >> 5;
  // A wave's 32 MFMA columns are HPW heads x RW rows: with G >= 8, two heads
  // of 16 rows, so a workgroup holds 16 rows of 8 heads (their K/V tiles are
  // staged once for all 8, and the selection union spans 16 rows); otherwise
  // one head of 32 rows per wave, the waves over the group's heads and then
  // over consecutive row blocks.
  const int HPW = a.G >= 8 ? 2 : 1;       // heads per wave
  const int RW = 32 / HPW;                // rows per wave
  const int HW = min(a.G, 4 * HPW);       // heads per workgroup
  const int WPH = HW / HPW;               // waves across the heads
  const int RB = 4 / WPH;                 // RW-row blocks per workgroup
  const int WROWS = RB * RW;              // rows per workgroup
  const int nhc = (a.G + HW - 1) / HW;
  const int nqg = (a.L + WROWS - 1) / WROWS;
  const int per = a.B * a.Hkv * nhc;
  const int qg = nqg - 1 - (int)(blockIdx.x / per);    // the long (late) query groups first
  int rem = blockIdx.x % per;
  const int hc = rem % nhc;
  rem /= nhc;
  const int g = rem % a.Hkv, b = rem / a.Hkv;
  const int gs = a.ng > 1 ? g : 0;
  const int wh = wave % WPH, wr = wave / WPH;
  const int wr0 = qg * WROWS;                           // first row of the workgroup
  const int r0 = wr0 + wr * RW;                         // first row of the wave
  const int hbase = hc * HW + wh * HPW;                 // the wave's first head within the group
  const bool active = wr < RB && hbase < a.G && r0 < a.L;
  // this lane's column: head hbase + ln / RW, row r0 + ln % RW
  const int hlane = hbase + ln / RW;
  const int hq = g * a.G + hlane;
  const int qi = r0 + ln % RW;
  const bool rowok = active && hlane < a.G && qi < a.L;
  const int nrb16 = (a.L + 15) / 16;
  const int rb0 = wr0 / 16;
  const int nrbw = min(WROWS / 16, nrb16 - rb0);

  // this lane's query row as B operand of S^T = K Q^T and dP^T = V dO^T
  bw_u32x4 qf[NC], dof[NC];
  float lse2 = kNegInf, dd = 0.f;
  {
    const int ii = rowok ? qi : 0, hh2 = rowok ? hq : 0;
    const int64_t oq = (int64_t)b * a.q_sb + (int64_t)ii * a.q_st + (int64_t)hh2 * a.q_sh + 8 * hh;
    const int64_t od = (int64_t)b * a.do_sb + (int64_t)ii * a.do_st + (int64_t)hh2 * a.do_sh + 8 * hh;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      qf[c] = rowok ? *(const bw_u32x4*)(a.q + oq + 16 * c) : zero4();
      dof[c] = rowok ? *(const bw_u32x4*)(a.dO + od + 16 * c) : zero4();
    }
    if (rowok) {
      const int64_t o = ((int64_t)b * a.Hq + hq) * a.L + qi;
      lse2 = a.lse[o] * kLog2e;
      dd = a.Dd[o];
    }
  }
  f32x16 dq_acc[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int i = 0; i < 16; ++i) dq_acc[t][i] = 0.f;

  const int wr1 = min(a.L, wr0 + WROWS) - 1;             // last row of the workgroup
  const int c_hi = min(wr1 / 64, (a.Lk - 1) / 64);
  int c = -1, wi = -1;
  uint32_t bits = 0u;
  if (MODE == BW_WINDOW) c = max(0, wr0 - a.window + 1) / 64 - 1;
  bool have = next_key_tile<MODE>(a, gs, b, nrb16, rb0, nrbw, c_hi, bits, wi, c);

  // staging item e = tid + 256p: keys 2kp, 2kp+1 of the tile (kp = e % 32), 16-byte chunk e / 32
  bw_u32x4 pk[NPASS][2], pv[NPASS][2];
  uint32_t pbits = 0u;
  auto issue = [&](int ct) {
    const int kc0 = ct * 64;
#pragma unroll
    for (int p = 0; p < NPASS; ++p) {
      const int e = tid + 256 * p, kp = e & 31, ch = e >> 5;
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int key = kc0 + 2 * kp + u;
        const bool ok = key < a.Lk;
        const int64_t o = (int64_t)b * a.k_sb + (int64_t)(ok ? key : 0) * a.k_st + (int64_t)g * a.k_sh + 8 * ch;
        pk[p][u] = ok ? *(const bw_u32x4*)(a.k + o) : zero4();
        pv[p][u] = ok ? *(const bw_u32x4*)(a.v + o) : zero4();
      }
    }
    if (MODE == BW_BLOCK)
      pbits = rowok ? a.rowbits[((int64_t)(gs * a.B + b) * a.nwords + (ct >> 5)) * a.L + qi] : 0u;
  };
  if (have) issue(c);

  while (have) {
    const int cur = c;
    __syncthreads();
#pragma unroll
    for (int p = 0; p < NPASS; ++p) {
      const int e = tid + 256 * p, kp = e & 31, ch = e >> 5;
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        *(bw_u32x4*)&s_k[(2 * kp + u) * RS + 8 * ch] = pk[p][u];
        *(bw_u32x4*)&s_v[(2 * kp + u) * RS + 8 * ch] = pv[p][u];
      }
      store_t8x2<TS>(s_kt, kp, ch, pk[p][0], pk[p][1]);
    }
    const bool selbit = MODE == BW_BLOCK ? ((pbits >> (cur & 31)) & 1u) != 0u : true;
    __syncthreads();
    have = next_key_tile<MODE>(a, gs, b, nrb16, rb0, nrbw, c_hi, bits, wi, c);
    if (have) issue(c);

    const int kc0 = cur * 64;
    bool any = active && kc0 <= r0 + RW - 1;
    if (MODE == BW_WINDOW) any = any && kc0 + 63 > r0 - a.window;
    if (MODE == BW_BLOCK) any = any && __ballot(selbit && rowok) != 0ull;
    if (any) {
      f32x16 s[2], dp[2];
#pragma unroll
      for (int kh = 0; kh < 2; ++kh)
#pragma unroll
        for (int i = 0; i < 16; ++i) { s[kh][i] = 0.f; dp[kh][i] = 0.f; }
#pragma unroll
      for (int kh = 0; kh < 2; ++kh)
#pragma unroll
        for (int c2 = 0; c2 < NC; ++c2) {
          const bw_u32x4 ak = *(const bw_u32x4*)&s_k[(32 * kh + ln) * RS + 16 * c2 + 8 * hh];
          const bw_u32x4 av = *(const bw_u32x4*)&s_v[(32 * kh + ln) * RS + 16 * c2 + 8 * hh];
          s[kh] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bwf(ak), bwf(qf[c2]), s[kh], 0, 0, 0);
          dp[kh] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bwf(av), bwf(dof[c2]), dp[kh], 0, 0, 0);
        }
      // element (kh, i): key kc0 + 32kh + 8(i/4) + 4hh + i%4, query row qi (this lane)
      // a tile every row of the wave sees whole skips the per-element test
      bool full = kc0 + 63 <= r0 && r0 + RW - 1 < a.L && kc0 + 63 < a.Lk && __ballot(!rowok) == 0ull;
      if (MODE == BW_WINDOW) full = full && kc0 > r0 + RW - 1 - a.window;
      if (MODE == BW_BLOCK) full = full && __ballot(!selbit) == 0ull;
      float ds[32];
      if (full) {
#pragma unroll
        for (int kh = 0; kh < 2; ++kh)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const float pvv = __builtin_amdgcn_exp2f(fmaf(s[kh][i], a.scale_log2, -lse2));
            ds[16 * kh + i] = pvv * (dp[kh][i] - dd);
          }
      } else {
#pragma unroll
        for (int kh = 0; kh < 2; ++kh)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int key = kc0 + 32 * kh + 8 * (i >> 2) + 4 * hh + (i & 3);
            const bool vis = bw_visible<MODE>(qi, key, a.L, a.Lk, a.window, selbit) && lse2 != kNegInf;
            const float pvv = vis ? __builtin_amdgcn_exp2f(fmaf(s[kh][i], a.scale_log2, -lse2)) : 0.f;
            ds[16 * kh + i] = pvv * (dp[kh][i] - dd);
          }
      }
      // dQ += dS K: k-slot 8hh + j of chunk kc is key 16kc + 8(j/4) + 4hh + j%4, i.e. value 8kc + j
#pragma unroll
      for (int kc = 0; kc < 4; ++kc) {
        const bw_u32x4 da = pack8(ds + 8 * kc);
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          const uint16_t* tk = &s_kt[(32 * t + ln) * TS + 16 * kc + 4 * hh];
          const bw_u32x4 bk = cat2(*(const bw_u32x2*)(tk), *(const bw_u32x2*)(tk + 8));
          dq_acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bwf(da), bwf(bk), dq_acc[t], 0, 0, 0);
        }
      }
    }
  }

  // dQ in C layout: lane (ln, hh) holds d = 32t + ln of columns m = 8(i/4) + 4hh + i%4,
  // i.e. head hbase + m / RW, row r0 + m % RW
  if (active) {
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int m = 8 * (i >> 2) + 4 * hh + (i & 3);
        const int row = r0 + m % RW, hm = hbase + m / RW;
        if (row >= a.L || hm >= a.G) continue;
        const int64_t o = (int64_t)b * a.dq_sb + (int64_t)row * a.dq_st + (int64_t)(g * a.G + hm) * a.dq_sh + 32 * t + ln;
        const float v = dq_acc[t][i] * a.scale;
        if (a.acc_q) a.dq[o] += v;
        else a.dq[o] = v;
      }
  }
}

// ---------------------------------------------------------------------------
// per-row preparation kernels (16 lanes per (b, i, h) row, 8 values per lane)
// ---------------------------------------------------------------------------
__device__ __forceinline__ void load8f(const void* p, int64_t off, int f32, float (&x)[8]) {
  if (f32) {
    const f32x4 u = *(const f32x4*)((const float*)p + off);
    const f32x4 w = *(const f32x4*)((const float*)p + off + 4);
#pragma unroll
    for (int j = 0; j < 4; ++j) { x[j] = u[j]; x[4 + j] = w[j]; }
  } else {
    const bw_u32x4 u = *(const bw_u32x4*)((const uint16_t*)p + off);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      x[2 * j] = bf16_to_f32((uint16_t)(u[j] & 0xffffu));
      x[2 * j + 1] = bf16_to_f32((uint16_t)(u[j] >> 16));
    }
  }
}

__device__ __forceinline__ float sum16(float v) {
  v += __shfl_xor(v, 8);
  v += __shfl_xor(v, 4);
  v += __shfl_xor(v, 2);
  v += __shfl_xor(v, 1);
  return v;
}

__global__ __launch_bounds__(256) void bwd_prep_full_kernel(BwdPrepArgs a) {
  const int64_t r = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);
  const int ch = threadIdx.x & 15;
  const int64_t nrow = (int64_t)a.B * a.L * a.Hq;
  if (r >= nrow) return;
  const int h = (int)(r % a.Hq);
  const int64_t bi = r / a.Hq;
  const int i = (int)(bi % a.L), b = (int)(bi / a.L);
  float acc = 0.f;
  if (8 * ch < a.D) {
    float x[8], y[8];
    load8f(a.dO, (int64_t)b * a.do_sb + (int64_t)i * a.do_st + (int64_t)h * a.do_sh + 8 * ch, a.do_f32, x);
    load8f(a.o, (int64_t)b * a.o_sb + (int64_t)i * a.o_st + (int64_t)h * a.o_sh + 8 * ch, a.o_f32, y);
#pragma unroll
    for (int j = 0; j < 8; ++j) acc = fmaf(x[j], y[j], acc);
  }
  acc = sum16(acc);
  if (ch == 0) a.Dd[((int64_t)b * a.Hq + h) * a.L + i] = acc;
}

__global__ __launch_bounds__(256) void bwd_prep_gate_kernel(BwdGateArgs a) {
  const int64_t r = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);
  const int ch = threadIdx.x & 15;
  const int64_t nrow = (int64_t)a.B * a.L * a.Hq;
  if (r >= nrow) return;
  const int h = (int)(r % a.Hq);
  const int64_t bi = r / a.Hq;
  const int i = (int)(bi % a.L), b = (int)(bi / a.L);
  const bool lane_on = 8 * ch < a.D;
  float dov[8], osp[8], ow[8], w[8], qv[8];
  float z = 0.f, sa = 0.f, sb = 0.f;
  if (lane_on) {
    load8f(a.dO, (int64_t)b * a.do_sb + (int64_t)i * a.do_st + (int64_t)h * a.do_sh + 8 * ch, a.do_f32, dov);
    load8f(a.osp, (int64_t)b * a.osp_sb + (int64_t)i * a.osp_st + (int64_t)h * a.osp_sh + 8 * ch, a.osp_f32, osp);
    load8f(a.ow, (int64_t)b * a.ow_sb + (int64_t)i * a.ow_st + (int64_t)h * a.ow_sh + 8 * ch, a.ow_f32, ow);
    load8f(a.q, (int64_t)b * a.q_sb + (int64_t)i * a.q_st + (int64_t)h * a.q_sh + 8 * ch, 0, qv);
    load8f(a.gate_w, (int64_t)h * a.D + 8 * ch, 1, w);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      z = fmaf(qv[j], w[j], z);
      sa = fmaf(dov[j], osp[j], sa);
      sb = fmaf(dov[j], ow[j], sb);
    }
  }
  z = sum16(z);
  sa = sum16(sa);
  sb = sum16(sb);
  if (a.gate_b) z += a.gate_b[h];
  const float gt = 1.f / (1.f + __expf(-z));
  const int64_t rl = ((int64_t)b * a.Hq + h) * a.L + i;
  const bool on = a.lse_sp[rl] != kNegInf;
  const float ge = on ? gt : 0.f;
  const float dz = on ? gt * (1.f - gt) * (sa - sb) : 0.f;
  if (lane_on) {
    const int64_t oc = (((int64_t)b * a.L + i) * a.Hq + h) * a.D + 8 * ch;
    bw_u32x4 us, uw;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      us[j] = pack_bf16x2(ge * dov[2 * j], ge * dov[2 * j + 1]);
      uw[j] = pack_bf16x2((1.f - ge) * dov[2 * j], (1.f - ge) * dov[2 * j + 1]);
    }
    *(bw_u32x4*)(a.do_sp + oc) = us;
    *(bw_u32x4*)(a.do_w + oc) = uw;
    float* dq = a.dq + (int64_t)b * a.dq_sb + (int64_t)i * a.dq_st + (int64_t)h * a.dq_sh + 8 * ch;
    const f32x4 lo = {dz * w[0], dz * w[1], dz * w[2], dz * w[3]};
    const f32x4 hi = {dz * w[4], dz * w[5], dz * w[6], dz * w[7]};
    *(f32x4*)dq = lo;
    *(f32x4*)(dq + 4) = hi;
  }
  if (ch == 0) {
    a.Dd_sp[rl] = ge * sa;
    a.Dd_w[rl] = (1.f - ge) * sb;
    a.dz[rl] = dz;
  }
}

// dgate_w and dgate_b partial sums: workgroup (h, split) sums rows split,
// split + nsplit, ...; part holds [kGateSplit][Hq][D] for w, then
// [kGateSplit][Hq] for the bias (the row sum of dz)
constexpr int kGateSplit = 64;

__global__ __launch_bounds__(256) void bwd_gate_partial_kernel(const float* dz, const uint16_t* q, int64_t q_sb,
                                                               int64_t q_st, int64_t q_sh, int B, int L, int Hq,
                                                               int D, float* part) {
  __shared__ float red[256];
  const int h = blockIdx.x % Hq, split = blockIdx.x / Hq;
  const int d = threadIdx.x % D, rg = threadIdx.x / D, nrg = 256 / D;
  __shared__ float redz[256];
  const int64_t n = (int64_t)B * L;
  float acc = 0.f, zs = 0.f;
  for (int64_t r = (int64_t)split * nrg + rg; r < n; r += (int64_t)kGateSplit * nrg) {
    const int b = (int)(r / L), i = (int)(r - (int64_t)b * L);
    const float z = dz[((int64_t)b * Hq + h) * L + i];
    acc = fmaf(z, bf16_to_f32(q[(int64_t)b * q_sb + (int64_t)i * q_st + (int64_t)h * q_sh + d]), acc);
    zs += z;
  }
  red[threadIdx.x] = acc;
  redz[threadIdx.x] = zs;
  __syncthreads();
  if (rg == 0) {
    for (int k = 1; k < nrg; ++k) acc += red[k * D + d];
    part[((int64_t)split * Hq + h) * D + d] = acc;
    if (d == 0) {
      for (int k = 1; k < nrg; ++k) zs += redz[k * D];
      part[(int64_t)kGateSplit * Hq * D + (int64_t)split * Hq + h] = zs;
    }
  }
}

__global__ __launch_bounds__(256) void bwd_gate_reduce_kernel(const float* part, int Hq, int D, float* out_w,
                                                              float* out_b) {
  const int e = blockIdx.x * 256 + threadIdx.x;
  if (e < Hq * D) {
    float s = 0.f;
    for (int k = 0; k < kGateSplit; ++k) s += part[(int64_t)k * Hq * D + e];
    out_w[e] = s;
  } else if (out_b && e < Hq * D + Hq) {
    const int h = e - Hq * D;
    const float* pb = part + (int64_t)kGateSplit * Hq * D;
    float s = 0.f;
    for (int k = 0; k < kGateSplit; ++k) s += pb[(int64_t)k * Hq + h];
    out_b[h] = s;
  }
}

__global__ __launch_bounds__(256) void bwd_selbits_kernel(const int32_t* idx, int64_t idx_sg, int64_t idx_sb,
                                                          int64_t idx_sr, int k, int ng, int B, int L, int nblk,
                                                          int nwords, uint32_t* rowbits, uint32_t* tilebits16) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t n = (int64_t)ng * B * L * k;
  if (e >= n) return;
  const int j = (int)(e % k);
  int64_t t = e / k;
  const int i = (int)(t % L);
  t /= L;
  const int b = (int)(t % B), gs = (int)(t / B);
  const int c = idx[gs * idx_sg + b * idx_sb + (int64_t)i * idx_sr + j];
  if (c < 0 || c >= nblk) return;
  const uint32_t bit = 1u << (c & 31);
  atomicOr(&rowbits[((int64_t)(gs * B + b) * nwords + (c >> 5)) * L + i], bit);
  atomicOr(&tilebits16[((int64_t)(gs * B + b) * ((L + 15) / 16) + (i >> 4)) * nwords + (c >> 5)], bit);
}

// Row list of 64-key block c of selection set gb (= gs * B + b): the rows
// i >= 64 c, ascending, whose bitmap holds block c, and their count.  One
// workgroup per (gb, c); thread t takes rows base + 16t .. base + 16t + 15 of
// each 4096-row pass, so thread order is row order and an exclusive scan of
// the per-thread counts places every row.
__global__ __launch_bounds__(256) void bwd_rowlist_kernel(const uint32_t* rowbits, int L, int nblk, int nwords,
                                                          int32_t* rowlist, int32_t* rowcnt) {
  __shared__ int s_tot[4];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int c = (int)(blockIdx.x % nblk);
  const int64_t gb = blockIdx.x / nblk;
  const int k0 = c * 64, sh = c & 31;
  const uint32_t* bits = rowbits + (gb * nwords + (c >> 5)) * (int64_t)L;
  int32_t* out = rowlist + (gb * nblk + c) * (int64_t)L;
  int carry = 0;
  for (int base = k0; base < L; base += 256 * 16) {
    const int r0 = base + 16 * tid;
    uint32_t wv[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) wv[j] = bits[min(r0 + j, L - 1)];
    uint32_t f = 0u;
#pragma unroll
    for (int j = 0; j < 16; ++j) f |= (r0 + j < L && ((wv[j] >> sh) & 1u) != 0u) ? (1u << j) : 0u;
    const int n = __popc(f);
    const int incl = wave_incl_scan_i32(n);
    __syncthreads();                      // the previous pass's totals are read
    if (lane == 63) s_tot[w] = incl;
    __syncthreads();
    int pos = carry + incl - n;
    for (int i = 0; i < w; ++i) pos += s_tot[i];
    carry += s_tot[0] + s_tot[1] + s_tot[2] + s_tot[3];
#pragma unroll
    for (int j = 0; j < 16; ++j)
      if ((f >> j) & 1u) out[pos++] = r0 + j;
  }
  if (tid == 0) rowcnt[gb * nblk + c] = carry;
}

template <int MODE, int D>
hipError_t dkdv_one(const BwdArgs& a, hipStream_t s) {
  const int tw = MODE == BW_CAUSAL ? 128 : 64;
  const int64_t grid = (int64_t)((a.Lk + tw - 1) / tw) * a.Hkv * a.B * a.nsplit;
  if constexpr (MODE == BW_CAUSAL)
    hipLaunchKernelGGL((bwd_dkdv_causal_kernel<MODE, D>), dim3((unsigned)grid), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((bwd_dkdv_kernel<MODE, D>), dim3((unsigned)grid), dim3(256), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.nsplit == 1) return e;
  const int64_t n = (int64_t)a.B * a.Lk * a.Hkv * (D / 4);
  hipLaunchKernelGGL(bwd_kv_reduce_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, a, D, tw);
  return hipGetLastError();
}

template <int MODE, int D>
hipError_t dq_one(const BwdArgs& a, hipStream_t s) {
  const int HPW = a.G >= 8 ? 2 : 1, HW = std::min(a.G, 4 * HPW), WROWS = (4 / (HW / HPW)) * (32 / HPW);
  const int nhc = (a.G + HW - 1) / HW;
  const int64_t grid = (int64_t)((a.L + WROWS - 1) / WROWS) * nhc * a.Hkv * a.B;
  hipLaunchKernelGGL((bwd_dq_kernel<MODE, D>), dim3((unsigned)grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace

// Rows per split: 64 row blocks (2048 rows) per workgroup, or more to keep at most 16
// splits.  The window branch's 64-key blocks are seen by at most 63 + window
// rows and are never split.
int bwd_dkdv_plan(int mode, int L, int window, int* split_rb) {
  const int nrb = (L + 31) / 32;
  int srb = 64;
  if ((nrb + srb - 1) / srb > 16) srb = (nrb + 15) / 16;
  if (mode == BW_WINDOW || nrb <= srb) { *split_rb = nrb > 0 ? nrb : 1; return 1; }
  *split_rb = srb;
  return (nrb + srb - 1) / srb;
}
// (causal: absolute row ranges, so a key tile's first split is the one holding
// its first row block and the earlier ones are empty; window and block-sparse:
// ranges of a block's rows counted from its first row)

size_t bwd_dkdv_ws_bytes(int nsplit, int B, int Lk, int Hkv, int D) {
  if (nsplit <= 1) return 0;
  const size_t part = (size_t)nsplit * B * Lk * Hkv * D * sizeof(float);
  // one flag per workgroup: 64-key workgroups (block-sparse) bound the count
  const size_t flags = (size_t)((Lk + 63) / 64) * Hkv * B * nsplit * sizeof(int32_t);
  return 2 * ((part + 255) & ~(size_t)255) + ((flags + 255) & ~(size_t)255);
}

void bwd_dkdv_bind_ws(BwdArgs& a, void* ws, int D) {
  if (a.nsplit <= 1) { a.part_k = a.part_v = nullptr; a.flags = nullptr; return; }
  const size_t part = (size_t)a.nsplit * a.B * a.Lk * a.Hkv * D * sizeof(float);
  const size_t pu = (part + 255) & ~(size_t)255;
  char* w = (char*)ws;
  a.part_k = (float*)w;
  a.part_v = (float*)(w + pu);
  a.flags = (int32_t*)(w + 2 * pu);
}

hipError_t launch_bwd_dkdv(int mode, int D, const BwdArgs& a, hipStream_t s) {
  if (a.L == 0 || a.Lk == 0) return hipSuccess;
  if (D == 128) {
    if (mode == BW_CAUSAL) return dkdv_one<BW_CAUSAL, 128>(a, s);
    if (mode == BW_WINDOW) return dkdv_one<BW_WINDOW, 128>(a, s);
    if (mode == BW_BLOCK) return dkdv_one<BW_BLOCK, 128>(a, s);
  } else if (D == 64) {
    if (mode == BW_CAUSAL) return dkdv_one<BW_CAUSAL, 64>(a, s);
    if (mode == BW_WINDOW) return dkdv_one<BW_WINDOW, 64>(a, s);
    if (mode == BW_BLOCK) return dkdv_one<BW_BLOCK, 64>(a, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_bwd_dq(int mode, int D, const BwdArgs& a, hipStream_t s) {
  if (a.L == 0 || a.Lk == 0) return hipSuccess;
  if (D == 128) {
    if (mode == BW_CAUSAL) return dq_one<BW_CAUSAL, 128>(a, s);
    if (mode == BW_WINDOW) return dq_one<BW_WINDOW, 128>(a, s);
    if (mode == BW_BLOCK) return dq_one<BW_BLOCK, 128>(a, s);
  } else if (D == 64) {
    if (mode == BW_CAUSAL) return dq_one<BW_CAUSAL, 64>(a, s);
    if (mode == BW_WINDOW) return dq_one<BW_WINDOW, 64>(a, s);
    if (mode == BW_BLOCK) return dq_one<BW_BLOCK, 64>(a, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_bwd_prep_full(const BwdPrepArgs& a, hipStream_t s) {
  const int64_t n = (int64_t)a.B * a.L * a.Hq;
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(bwd_prep_full_kernel, dim3((unsigned)((n + 15) / 16)), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_bwd_prep_gate(const BwdGateArgs& a, hipStream_t s) {
  const int64_t n = (int64_t)a.B * a.L * a.Hq;
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(bwd_prep_gate_kernel, dim3((unsigned)((n + 15) / 16)), dim3(256), 0, s, a);
  return hipGetLastError();
}

size_t bwd_gate_partial_floats(int Hq, int D) { return (size_t)kGateSplit * Hq * (D + 1); }

hipError_t launch_bwd_gate_grad(const float* dz, const uint16_t* q, int64_t q_sb, int64_t q_st, int64_t q_sh,
                                int B, int L, int Hq, int D, float* part, float* dgate_w, float* dgate_b,
                                hipStream_t s) {
  hipLaunchKernelGGL(bwd_gate_partial_kernel, dim3((unsigned)(Hq * kGateSplit)), dim3(256), 0, s, dz, q, q_sb, q_st,
                     q_sh, B, L, Hq, D, part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(bwd_gate_reduce_kernel, dim3((unsigned)((Hq * D + Hq + 255) / 256)), dim3(256), 0, s, part, Hq,
                     D, dgate_w, dgate_b);
  return hipGetLastError();
}

hipError_t launch_bwd_selbits(const int32_t* idx, int64_t idx_sg, int64_t idx_sb, int64_t idx_sr, int k, int ng,
                              int B, int L, int nblk, int nwords, uint32_t* rowbits, uint32_t* tilebits16,
                              int32_t* rowlist, int32_t* rowcnt, hipStream_t s) {
  const int nrb16 = (L + 15) / 16;
  if (L == 0) return hipSuccess;
  hipError_t e = launch_fill_i32((int32_t*)rowbits, 0, (int64_t)ng * B * L * nwords, s);
  if (e != hipSuccess) return e;
  e = launch_fill_i32((int32_t*)tilebits16, 0, (int64_t)ng * B * nrb16 * nwords, s);
  if (e != hipSuccess) return e;
  const int64_t n = (int64_t)ng * B * L * k;
  if (n > 0) {
    hipLaunchKernelGGL(bwd_selbits_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, idx, idx_sg, idx_sb,
                       idx_sr, k, ng, B, L, nblk, nwords, rowbits, tilebits16);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  hipLaunchKernelGGL(bwd_rowlist_kernel, dim3((unsigned)((int64_t)ng * B * nblk)), dim3(256), 0, s,
                     (const uint32_t*)rowbits, L, nblk, nwords, rowlist, rowcnt);
  return hipGetLastError();
}

}  // namespace hys
