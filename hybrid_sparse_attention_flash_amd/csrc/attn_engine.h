// Tiled MFMA attention engine for the HySparse / HySparse2 prefill path (gfx950).
//
// One workgroup = 4 waves = 256 threads.  It owns a "row set": BQ consecutive
// queries x HC query heads that share one KV head (GQA/MQA), laid out
// query-major (row r = query r/HC, head r%HC), 32*NB rows per wave.  It walks a
// sequence of 64-key tiles -- contiguous (causal / window) or gathered (selected
// blocks / selected tokens) -- staging each tile through LDS:
//   K   as [64 keys][D]   (row padded), read as MFMA A fragments, and
//   V^T as [D][64 keys]   (row padded), transposed in registers on the way in,
// with fp8 e4m3 K/V decoded to bf16 while staging.  The logits are formed
// transposed, S^T = K Q^T (v_mfma_f32_32x32x16_bf16, or 32x32x2_f32 for fp32),
// so each lane holds one row's logits for 32 of the 64 keys and the row
// softmax needs a single cross-lane exchange; O^T = V^T P^T then consumes the
// probabilities straight from the logit registers.  Online softmax runs in the
// base-2 domain on raw dot products; the natural-unit scaled logit is recovered
// exactly where scores are emitted.
//
// Score emission (the full layer's byproduct, TechWalker HySparse write-up,
// paragraph on the modified FlashAttention kernel): the per-row tile maximum
// that the online softmax needs anyway is the block maximum when tiles are the
// 64-key blocks; the max over the query heads of a KV group is taken in LDS.
// For HySparse2 token scores the per-key maximum over a workgroup's rows is
// reduced across lanes (in registers) and waves (in LDS); the head chunks of a
// query tile run as separate workgroups and combine their maxima with an
// atomic max on order-preserving integer keys, which is exact and order
// independent, so results are deterministic.  The key array is cleared
// before and decoded to fp32 after the attention launch.
#pragma once
#include "common.h"
#include "kernels.h"
#include "block_union.h"
#include <type_traits>

namespace hys {

template <typename QT> struct Compute;
template <> struct Compute<float> { using CT = float; static constexpr int KPAD = 4; static constexpr int VPAD = 4; };
template <> struct Compute<uint16_t> { using CT = uint16_t; static constexpr int KPAD = 8; static constexpr int VPAD = 4; };

// ---------------------------------------------------------------------------
// the engine
// ---------------------------------------------------------------------------

template <int MODE, typename QT, typename KT, int D, int NB>
__global__ __launch_bounds__(256, (NB == 1) ? 2 : 1) void attn_tile_kernel(const AttnArgs a) {
  using CT = typename Compute<QT>::CT;
  constexpr bool F32 = sizeof(CT) == 4;
  constexpr int KROW = D + Compute<QT>::KPAD;      // LDS row stride of K (elements)
  constexpr int VROW = 64 + Compute<QT>::VPAD;     // LDS row stride of V^T (elements)
  constexpr int ROWS = 4 * 32 * NB;                // rows per workgroup
  constexpr int KUN = 64 * (D / 8);                // K staging units (8 elements each)
  constexpr int KU = KUN / 256;
  constexpr int VUN = 16 * (D / 8);                // V staging units (4 keys x 8 d)
  constexpr int VU = (VUN + 255) / 256;
  constexpr int NDB = D / 32;                      // 32-wide d blocks of O^T
  constexpr int NQC = F32 ? D / 2 : D / 16;        // Q fragments per row (k-steps of S^T)
  constexpr int UMAX = 4 * ROWS;                   // max union entries (block mode)
  constexpr int NBWMAX = 512;                      // max bitmap words (block mode)
  constexpr int TLMAX = 2048;                      // max token-list length (token mode)
  static_assert(KUN % 256 == 0, "D must be 64 or 128");
  // modes whose tiles include selected key blocks
  constexpr bool BLOCKSEL = MODE == M_SPARSE_BLOCK || MODE == M_SPARSE_SWA;

  // two stages: tile n is consumed from one while tile n+1 is written to the other
  __shared__ __attribute__((aligned(16))) CT Klds[2 * 64 * KROW];
  __shared__ __attribute__((aligned(16))) CT VTlds[2 * D * VROW];
  __shared__ __attribute__((aligned(16))) int kinfo[2 * 64];
  constexpr int RS = ROWS > 256 ? ROWS : 256;      // stride of the two score-reduction halves
  __shared__ __attribute__((aligned(16))) float red[2 * RS];
  __shared__ int s_misc[4];
  // block-sparse lists
  __shared__ uint32_t s_bitmap[BLOCKSEL ? NBWMAX : 1];
  __shared__ int s_wpre[BLOCKSEL ? NBWMAX : 1];
  __shared__ int s_ulist[BLOCKSEL ? UMAX : 1];
  __shared__ unsigned long long s_member[BLOCKSEL ? UMAX : 1];
  // token-sparse lists
  __shared__ int s_tlist[(MODE == M_SPARSE_TOKEN) ? TLMAX : 1];
  __shared__ unsigned char s_selw[(MODE == M_SPARSE_TOKEN) ? 2048 : 1];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6, hh = lane >> 5, ln = lane & 31;

  int bid = blockIdx.x;
  if (bid >= a.grid_used) return;

  // ---- work decomposition ------------------------------------------------
  int b, qt, g = 0, ch_begin = 0;
  if (MODE == M_FULL_TILE || MODE == M_SPARSE_TOKEN) {
    // the head chunks of one query tile run back to back on one XCD
    // (workgroups are dealt to the 8 XCDs round robin), so they stream the
    // same K/V tiles through its L2 at about the same time
    const int nch = a.Hkv * a.nhc;
    const int xcd = bid & 7, slot = bid >> 3;
    const int ch = slot % nch;
    const int tile_rank = (slot / nch) * 8 + xcd;
    b = tile_rank % a.B;
    qt = tile_rank / a.B;
    if (qt >= a.ntq) return;
    if (MODE == M_FULL_TILE) qt = a.ntq - 1 - qt;  // causal: longest rows first
    ch_begin = ch;
  } else {
    g = bid % a.Hkv;                               // KV group fastest: XCD x sees groups x mod Hkv
    const int rest = bid / a.Hkv;
    b = rest % a.B;
    qt = a.ntq - 1 - rest / a.B;
  }
  const int q0 = qt * a.BQ;
  const int q_last = min(q0 + a.BQ, a.Lq) - 1;
  // absolute positions (row r of this call is position q_off + r): every
  // causal and window range below is in absolute positions, rows address
  // q, o and lse relative to the call
  const int qa0 = q0 + a.q_off, qa_last = q_last + a.q_off;
  const int HC = a.HC;
  // block scores reduced inside each wave when a query's heads are adjacent lanes
  const bool lane_scores = (MODE == M_FULL_BLOCK) && (32 % HC == 0);

  // the workgroup's head chunk; its Q fragments are loaded first, so their
  // latency overlaps the selection-list building below
  const int ch = ch_begin;
  int h0 = 0;
  if (MODE == M_FULL_TILE || MODE == M_SPARSE_TOKEN) { g = ch / a.nhc; h0 = (ch % a.nhc) * HC; }

  // ---- rows owned by this lane -------------------------------------------
  int qpos[NB], head[NB], qiv[NB];
  bool valid[NB];
  bool wave_full = true;
  int wave_qmin = 0x7fffffff, wave_qmax = -1;
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int r = wave * 32 * NB + nb * 32 + ln;
    const int qi = r / HC, hl = r - qi * HC;
    qiv[nb] = qi;
    qpos[nb] = q0 + qi;
    head[nb] = g * a.G + h0 + hl;
    valid[nb] = qi < a.BQ && qpos[nb] < a.Lq && (h0 + hl) < a.G;
  }
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    int qv = valid[nb] ? qpos[nb] : 0x7fffffff;
    int qx = valid[nb] ? qpos[nb] : -1;
    for (int o = 32; o >= 1; o >>= 1) { qv = min(qv, __shfl_xor(qv, o)); qx = max(qx, __shfl_xor(qx, o)); }
    wave_qmin = min(wave_qmin, qv);
    wave_qmax = max(wave_qmax, qx);
    wave_full = wave_full && (__ballot(!valid[nb]) == 0ull);
  }
  const bool wave_any = wave_qmax >= 0;
  unsigned long long wave_qmask = 0ull;
  if (BLOCKSEL) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      unsigned long long m = valid[nb] ? (1ull << qiv[nb]) : 0ull;
      for (int o = 32; o >= 1; o >>= 1) m |= __shfl_xor(m, o);
      wave_qmask |= m;
    }
  }

  // ---- Q fragments (B operand of S^T) ------------------------------------
  const QT* qbase = (const QT*)a.q + (int64_t)b * a.q_sb;
  typedef typename std::conditional<F32, float, bf16x8>::type QFrag;
  QFrag qf[NB][NQC];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    // unconditional loads from a clamped row (see keep_if), zeroed for padding rows
    const QT* qr = qbase + (valid[nb] ? (int64_t)qpos[nb] * a.q_st + (int64_t)head[nb] * a.q_sh : 0);
#pragma unroll
    for (int c = 0; c < NQC; ++c) {
      if constexpr (F32) {
        const float x = qr[2 * c + hh];
        qf[nb][c] = valid[nb] ? x : 0.0f;
      } else {
        const uint4 x = *(const uint4*)(qr + 16 * c + 8 * hh);
        const uint4 z = {0u, 0u, 0u, 0u};
        qf[nb][c] = as_bf16x8(valid[nb] ? x : z);
      }
    }
  }

  // ---- per-WG selection lists ----------------------------------------------
  int ntiles = 0;
  int kbase = 0;            // contiguous modes: first key
  int kend = 0;             // contiguous modes: last key (inclusive)
  int npre = 0, wstart = 0, wend = 0;
  int nsp = 0;              // M_SPARSE_SWA: tiles [0, nsp) are selected blocks, the rest the window
  if (MODE == M_FULL || MODE == M_FULL_BLOCK || MODE == M_FULL_TILE) {
    kbase = 0; kend = min(qa_last, a.Lk - 1);
    ntiles = kend / 64 + 1;
  } else if (MODE == M_SWA_GATE) {
    kbase = max(0, qa0 - a.window + 1); kend = min(qa_last, a.Lk - 1);
    ntiles = (kend - kbase + 1 + 63) / 64;
  } else if (BLOCKSEL) {
    const int32_t* ib = a.idx + (int64_t)b * a.idx_sb + (int64_t)g * a.idx_sg;
    ntiles = build_block_union<UMAX, NBWMAX>(ib, a.idx_sr, a.topk, q0, a.BQ, a.Lq, a.nblk, s_bitmap, s_wpre,
                                             s_ulist, s_member, &s_misc[0]);
    if (MODE == M_SPARSE_SWA) {
      // then the window [qa0 - window + 1, qa_last] of the layer's own K/V
      nsp = ntiles;
      wstart = max(0, qa0 - a.window + 1);
      wend = min(qa_last, a.Lk - 1);
      ntiles = nsp + (wend - wstart + 1 + 63) / 64;
    }
  } else if (MODE == M_SPARSE_TOKEN) {
    wstart = max(0, qa0 - a.window + 1);
    wend = min(qa_last, a.Lk - 1);
    const int nw = wend - wstart + 1;
    for (int x = tid; x < nw; x += 256) s_selw[x] = 0;
    __syncthreads();
    const int32_t* sel = a.idx + (int64_t)b * a.idx_sb + (int64_t)qt * a.idx_sr;
    // all of the tile's selections are loaded up front (one memory latency,
    // not one per round below); k <= TLMAX = 8 * 256
    int sv[TLMAX / 256];
#pragma unroll
    for (int i = 0; i < TLMAX / 256; ++i) {
      const int e = i * 256 + tid;
      sv[i] = (e < a.topk) ? sel[e] : -1;
    }
    // order-preserving compaction of the selected tokens that precede the window
    int carry = 0;
#pragma unroll
    for (int i = 0; i < TLMAX / 256; ++i) {
      if (i * 256 >= a.topk) break;
      const int s = sv[i];
      const bool pre = s >= 0 && s < wstart;
      if (s >= wstart && s <= wend) s_selw[s - wstart] = 1;
      const unsigned long long bal = __ballot(pre);
      if (lane == 0) s_misc[wave] = __popcll(bal);
      __syncthreads();
      int before = carry;
      for (int w = 0; w < wave; ++w) before += s_misc[w];
      const int mypos = before + __popcll(bal & ((1ull << lane) - 1ull));
      if (pre && mypos < TLMAX) s_tlist[mypos] = s;
      carry += s_misc[0] + s_misc[1] + s_misc[2] + s_misc[3];
      __syncthreads();
    }
    npre = min(carry, TLMAX);
    ntiles = (npre + nw + 63) / 64;
  }

  // ---- staging helpers -----------------------------------------------------
  const KT* kb = (const KT*)a.k + (int64_t)b * a.k_sb;
  const KT* vb = (const KT*)a.v + (int64_t)b * a.v_sb;
  // the layer's own window K/V (same strides as k, v)
  const KT* kwb = (MODE == M_SPARSE_SWA) ? (const KT*)a.kw + (int64_t)b * a.k_sb : kb;
  const KT* vwb = (MODE == M_SPARSE_SWA) ? (const KT*)a.vw + (int64_t)b * a.v_sb : vb;

  // key position of tile slot t of tile n; -1 when the slot is empty.
  // For the token mode, bit 30 flags a selected (as opposed to window-only) token.
  auto keypos = [&](int n, int t) __attribute__((always_inline)) -> int {
    if (MODE == M_SPARSE_SWA && n >= nsp) {
      const int j = wstart + (n - nsp) * 64 + t;
      return j <= wend ? j : -1;
    } else if (BLOCKSEL) {
      const int j = s_ulist[n] * 64 + t;
      return j < a.Lk ? j : -1;
    } else if (MODE == M_SPARSE_TOKEN) {
      const int p = n * 64 + t;
      if (p < npre) return s_tlist[p] | (1 << 30);
      const int j = wstart + (p - npre);
      if (j > wend) return -1;
      return s_selw[j - wstart] ? (j | (1 << 30)) : j;
    } else {
      const int j = kbase + n * 64 + t;
      return j <= kend ? j : -1;
    }
  };

  Raw8<KT> kreg[KU];
  Raw8<KT> vreg[VU][4];
  uint32_t kmask = 0u, vmask = 0u;     // staged units whose slot holds a key
  int my_kinfo = 0;

  // First key of tile n when its 64 slots are the consecutive keys j0..j0+63
  // (a full contiguous tile or a whole selected block): then one wave-uniform
  // base pointer serves every load and no slot needs masking.
  auto full_tile = [&](int n, int& j0) __attribute__((always_inline)) -> bool {
    if (MODE == M_SPARSE_TOKEN) { j0 = 0; return false; }
    if (MODE == M_SPARSE_SWA && n >= nsp) { j0 = wstart + (n - nsp) * 64; return j0 + 63 <= wend; }
    if (BLOCKSEL) { j0 = s_ulist[n] * 64; return j0 + 63 < a.Lk; }
    j0 = kbase + n * 64;
    return j0 + 63 <= kend;
  };
  // per-thread element offsets inside a tile (independent of the tile): unit
  // tid + 256u covers key tid/(D/8) + u*256/(D/8) (K) and, for V, key group
  // (tid%16) with d chunk tid/16 + 16u, so one base register per operand and
  // wave-uniform strides address every unit
  const int koff0 = (tid / (D / 8)) * (int)a.k_st + (tid % (D / 8)) * 8;
  const int kstep = (256 / (D / 8)) * (int)a.k_st;
  const int voff0 = ((tid % 16) * 4) * (int)a.v_st + (tid / 16) * 8;
  bool staged_full = true;

  auto stage_load = [&](int n, int g_) __attribute__((always_inline)) {
    const int kvh = g_;
    const bool own = MODE == M_SPARSE_SWA && n >= nsp;
    const KT* ksrc = own ? kwb : kb;
    const KT* vsrc = own ? vwb : vb;
    int j0;
    staged_full = __builtin_amdgcn_readfirstlane((int)full_tile(n, j0)) != 0;
    if (staged_full) {
      const KT* kt = ksrc + (int64_t)j0 * a.k_st + (int64_t)kvh * a.k_sh;
      const KT* vt = vsrc + (int64_t)j0 * a.v_st + (int64_t)kvh * a.v_sh;
#pragma unroll
      for (int u = 0; u < KU; ++u) kreg[u] = load8<KT>(kt + koff0 + u * kstep);
#pragma unroll
      for (int u = 0; u < VU; ++u)
        if (VUN % 256 == 0 || tid + 256 * u < VUN) {
#pragma unroll
          for (int r = 0; r < 4; ++r) vreg[u][r] = load8<KT>(vt + voff0 + r * (int)a.v_st + u * 128);
        }
      if (tid < 64) my_kinfo = j0 + tid;
      return;
    }
    kmask = 0u; vmask = 0u;
#pragma unroll
    for (int u = 0; u < KU; ++u) {
      const int unit = tid + 256 * u;
      const int key = unit / (D / 8), c8 = unit % (D / 8);
      const int kp = keypos(n, key);
      const int j = kp >= 0 ? (kp & ~(1 << 30)) : 0;
      kmask |= (kp >= 0 ? 1u : 0u) << u;
      kreg[u] = load8<KT>(ksrc + (int64_t)j * a.k_st + (int64_t)kvh * a.k_sh + c8 * 8);
    }
#pragma unroll
    for (int u = 0; u < VU; ++u) {
      const int unit = tid + 256 * u;
      if (VUN % 256 == 0 || unit < VUN) {
        const int kg = unit % 16, dc = unit / 16;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int kp = keypos(n, kg * 4 + r);
          const int j = kp >= 0 ? (kp & ~(1 << 30)) : 0;
          vmask |= (kp >= 0 ? 1u : 0u) << (4 * u + r);
          vreg[u][r] = load8<KT>(vsrc + (int64_t)j * a.v_st + (int64_t)kvh * a.v_sh + dc * 8);
        }
      }
    }
    if (tid < 64) {
      const int kp = keypos(n, tid);
      my_kinfo = kp >= 0 ? kp : 0x3fffffff;   // empty slots are later than every query
    }
  };

  // Registers of the staged tile -> LDS stage `buf` (K row-major, V transposed).
  // Instantiated twice so that whole contiguous tiles store without any
  // per-unit masking; the choice is wave-uniform.
  auto stage_store_impl = [&](int buf, auto masked_tag) __attribute__((always_inline)) {
    constexpr bool MASKED = decltype(masked_tag)::value;
    CT* Kb = Klds + buf * (64 * KROW);
    CT* Vb = VTlds + buf * (D * VROW);
#pragma unroll
    for (int u = 0; u < KU; ++u) {
      const int unit = tid + 256 * u;
      const int key = unit / (D / 8), c8 = unit % (D / 8);
      if constexpr (MASKED) keep_if(kreg[u], (kmask >> u) & 1u);
      Cvt8<CT> c = to_ct(kreg[u]);
      CT* dst = &Kb[key * KROW + c8 * 8];
      *(uint4*)dst = c.a;
      if constexpr (F32) *(uint4*)(dst + 4) = c.b;
    }
#pragma unroll
    for (int u = 0; u < VU; ++u) {
      const int unit = tid + 256 * u;
      if (VUN % 256 == 0 || unit < VUN) {
        // the 16 lanes of one write cover the 16 key groups of one V^T row:
        // consecutive 8-byte slots, no bank conflicts
        const int kg = unit % 16, dc = unit / 16;
        if constexpr (MASKED) {
#pragma unroll
          for (int r = 0; r < 4; ++r) keep_if(vreg[u][r], (vmask >> (4 * u + r)) & 1u);
        }
        Cvt8<CT> r0 = to_ct(vreg[u][0]), r1 = to_ct(vreg[u][1]), r2 = to_ct(vreg[u][2]), r3 = to_ct(vreg[u][3]);
        if constexpr (!F32) {
#pragma unroll
          for (int p = 0; p < 4; ++p) {
            const uint32_t w0 = u4get(r0.a, p), w1 = u4get(r1.a, p), w2 = u4get(r2.a, p), w3 = u4get(r3.a, p);
            uint2 e, o;
            e.x = __builtin_amdgcn_perm(w1, w0, 0x05040100u); e.y = __builtin_amdgcn_perm(w3, w2, 0x05040100u);
            o.x = __builtin_amdgcn_perm(w1, w0, 0x07060302u); o.y = __builtin_amdgcn_perm(w3, w2, 0x07060302u);
            *(uint2*)&Vb[(dc * 8 + 2 * p) * VROW + kg * 4] = e;
            *(uint2*)&Vb[(dc * 8 + 2 * p + 1) * VROW + kg * 4] = o;
          }
        } else {
#pragma unroll
          for (int d = 0; d < 8; ++d) {
            uint4 t;
            t.x = d < 4 ? u4get(r0.a, d) : u4get(r0.b, d - 4);
            t.y = d < 4 ? u4get(r1.a, d) : u4get(r1.b, d - 4);
            t.z = d < 4 ? u4get(r2.a, d) : u4get(r2.b, d - 4);
            t.w = d < 4 ? u4get(r3.a, d) : u4get(r3.b, d - 4);
            *(uint4*)&Vb[(dc * 8 + d) * VROW + kg * 4] = t;
          }
        }
      }
    }
    if (tid < 64) kinfo[buf * 64 + tid] = my_kinfo;
  };
  auto stage_store = [&](int buf) __attribute__((always_inline)) {
    if (staged_full) stage_store_impl(buf, std::false_type{});
    else stage_store_impl(buf, std::true_type{});
  };


  {
    float m_run[NB], l_run[NB];
    f32x16 acc[NB][NDB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      m_run[nb] = kNegInf; l_run[nb] = 0.f;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[nb][db][i] = 0.f;
    }

    const float c2 = a.scale_log2;
    const float lazy_raw = kLazyLog2 / c2;    // the slack in raw dot-product units

    // M_SPARSE_SWA: at the first window tile, the sparse branch is finished.
    // Its normalised output goes to this row's output slot (read back by the
    // same lane in the epilogue) and the softmax state restarts for the window.
    bool sp_live[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) sp_live[nb] = false;
    auto finish_sparse_branch = [&]() __attribute__((always_inline)) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const float lsum = l_run[nb] + __shfl_xor(l_run[nb], 32);
        sp_live[nb] = m_run[nb] != kNegInf;
        const float inv = sp_live[nb] ? a.v_scale / lsum : 0.f;
        if (valid[nb]) {
          const int64_t row_off_o = (int64_t)b * a.o_sb + (int64_t)qpos[nb] * a.o_st + (int64_t)head[nb] * a.o_sh;
#pragma unroll
          for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int i4 = 0; i4 < 4; ++i4) {
              const int d = db * 32 + 8 * i4 + 4 * hh;
              const f32x16& ac = acc[nb][db];
              if (a.o_f32) {
                float4 out = {ac[4 * i4] * inv, ac[4 * i4 + 1] * inv, ac[4 * i4 + 2] * inv, ac[4 * i4 + 3] * inv};
                *(float4*)((float*)a.o + row_off_o + d) = out;
              } else {
                uint2 out;
                out.x = pack_bf16x2(ac[4 * i4] * inv, ac[4 * i4 + 1] * inv);
                out.y = pack_bf16x2(ac[4 * i4 + 2] * inv, ac[4 * i4 + 3] * inv);
                *(uint2*)((uint16_t*)a.o + row_off_o + d) = out;
              }
            }
        }
        m_run[nb] = kNegInf; l_run[nb] = 0.f;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int i = 0; i < 16; ++i) acc[nb][db][i] = 0.f;
      }
    };

    // score emission for tile n (reads red[n & 1]); called by all threads after a barrier
    auto emit_scores = [&](int n) __attribute__((always_inline)) {
      if (MODE == M_FULL_BLOCK && !lane_scores) {
        const float* rb = red + (n & 1) * RS;
        float* sc = a.scores + (int64_t)g * a.sc_sg + (int64_t)b * a.sc_sb;
        for (int t = tid; t < a.BQ; t += 256) {
          const int q = q0 + t;
          if (q < a.Lq) {
            float mx = kNegInf;
            for (int hl = 0; hl < HC; ++hl) mx = fmaxf(mx, rb[t * HC + hl]);
            sc[(int64_t)q * a.sc_sr + n] = mx * a.logit_scale;
          }
        }
      } else if (MODE == M_FULL_TILE) {
        if (tid < 64) {
          const float* rb = red + (n & 1) * RS;
          float mx = fmaxf(fmaxf(rb[tid], rb[64 + tid]), fmaxf(rb[128 + tid], rb[192 + tid]));
          const int j = n * 64 + tid;
          if (j < a.Lk) {
            // head chunks of the tile combine through an atomic max of
            // order-preserving keys: exact, and independent of their order
            uint32_t* dst = (uint32_t*)(a.scores + (int64_t)b * a.sc_sb + (int64_t)qt * a.sc_sr) + j;
            atomicMax(dst, f32_order_key(mx * a.logit_scale));
          }
        }
      }
    };

    // ---- tile loop ---------------------------------------------------------
    // One barrier per tile: tile n is read from stage n&1 while the registers
    // holding tile n+1 are written to the other stage and tile n+2 is fetched.
    if (ntiles > 0) {
      stage_load(0, g);
      stage_store(0);
      if (ntiles > 1) stage_load(1, g);
    }
    __syncthreads();
    for (int n = 0; n < ntiles; ++n) {
      if (MODE == M_SPARSE_SWA && n == nsp) finish_sparse_branch();
      const int cur = n & 1;
      const CT* Kc = Klds + cur * (64 * KROW);
      const CT* Vc = VTlds + cur * (D * VROW);
      const int* kic = kinfo + cur * 64;
      if (n > 0) emit_scores(n - 1);

      // wave-level skip: nothing of this tile is visible to any row of the wave
      bool active = wave_any;
      const bool sel_tile = BLOCKSEL && !(MODE == M_SPARSE_SWA && n >= nsp);
      const unsigned long long memb = sel_tile ? s_member[n] : 0ull;
      if (sel_tile) active = active && ((memb & wave_qmask) != 0ull);

      if (!active) {
        if (MODE == M_FULL_BLOCK && hh == 0) {
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) {
            if (lane_scores) {
              if (valid[nb] && (ln % HC) == 0)
                a.scores[(int64_t)g * a.sc_sg + (int64_t)b * a.sc_sb + (int64_t)qpos[nb] * a.sc_sr + n] = kNegInf;
            } else {
              red[(n & 1) * RS + wave * 32 * NB + nb * 32 + ln] = kNegInf;
            }
          }
        }
        if (MODE == M_FULL_TILE) red[(n & 1) * RS + wave * 64 + lane] = kNegInf;
      } else {
        // S^T = K Q^T  (M = 64 keys as two 32-blocks, N = rows, K = D); the K
        // fragments of step c+1 are read while the MFMAs of step c issue
        f32x16 s[2][NB];
        const f32x16 zero16 = {};
        if constexpr (F32) {
          float kn0 = Kc[ln * KROW + hh], kn1 = Kc[(32 + ln) * KROW + hh];
#pragma unroll
          for (int c = 0; c < NQC; ++c) {
            const float k0 = kn0, k1 = kn1;
            if (c + 1 < NQC) { kn0 = Kc[ln * KROW + 2 * (c + 1) + hh]; kn1 = Kc[(32 + ln) * KROW + 2 * (c + 1) + hh]; }
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
              s[0][nb] = __builtin_amdgcn_mfma_f32_32x32x2f32(k0, qf[nb][c], c == 0 ? zero16 : s[0][nb], 0, 0, 0);
              s[1][nb] = __builtin_amdgcn_mfma_f32_32x32x2f32(k1, qf[nb][c], c == 0 ? zero16 : s[1][nb], 0, 0, 0);
            }
          }
        } else {
          // K fragments are read two k-steps ahead of the MFMAs that use them
          uint4 kf[NQC][2];
          auto kfrag = [&](int c) __attribute__((always_inline)) {
            kf[c][0] = *(const uint4*)&Kc[ln * KROW + 16 * c + 8 * hh];
            kf[c][1] = *(const uint4*)&Kc[(32 + ln) * KROW + 16 * c + 8 * hh];
          };
          kfrag(0);
          kfrag(1);
#pragma unroll
          for (int c = 0; c < NQC; ++c) {
            if (c + 2 < NQC) kfrag(c + 2);
            // keep the reads ahead: the scheduler would otherwise sink each
            // read next to its MFMA and expose the full LDS latency per step
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
              s[0][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(kf[c][0]), qf[nb][c], c == 0 ? zero16 : s[0][nb], 0, 0, 0);
              s[1][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(kf[c][1]), qf[nb][c], c == 0 ? zero16 : s[1][nb], 0, 0, 0);
            }
          }
        }

        // V^T fragments (A operand of O^T): the first d block is read now so
        // that its LDS latency hides under the softmax; later blocks are read
        // one d block ahead of their MFMAs
        typedef typename std::conditional<F32, float, uint4>::type VFrag;
        VFrag vf[F32 ? 1 : NDB][4];
        auto vfrag = [&](int db, int kc) __attribute__((always_inline)) {
          const CT* vr = &Vc[(db * 32 + ln) * VROW + 16 * kc + 4 * hh];
          const uint2 lo = *(const uint2*)vr;
          const uint2 hi = *(const uint2*)(vr + 8);
          uint4 va; va.x = lo.x; va.y = lo.y; va.z = hi.x; va.w = hi.y;
          return va;
        };
        if constexpr (!F32) {
#pragma unroll
          for (int kc = 0; kc < 4; ++kc) vf[0][kc] = vfrag(0, kc);
          __builtin_amdgcn_sched_barrier(0);
        }

        // Visibility.  Each lane's row sees the keys [lo, hi] of this tile
        // (causal, window), or none (invalid row, block not selected by its
        // query).  Rows that see nothing are excluded through the softmax
        // reference below, not element by element; element masks are applied
        // only when some row of the wave sees part of the tile.
        bool row_on[NB];
        unsigned vbase[NB], vspan[NB];
        // token mode: list slots before npre hold selected tokens that precede
        // the window start, hence every query of the tile; a tile made only of
        // them needs no element mask
        bool elem_mask = MODE == M_SPARSE_TOKEN && !(n * 64 + 63 < npre);
        {
          int jt0 = 0;
          if (MODE != M_SPARSE_TOKEN) full_tile(n, jt0);   // consecutive keys from jt0
          bool part = false, off_row = false;
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) {
            const bool win = MODE == M_SWA_GATE || (MODE == M_SPARSE_SWA && !sel_tile);
            const int hi = qpos[nb] + a.q_off;
            const int lo = win ? hi - a.window + 1 : 0;
            bool on = valid[nb];
            if (BLOCKSEL && sel_tile) on = on && ((memb >> qiv[nb]) & 1ull) != 0ull;
            row_on[nb] = on;
            vbase[nb] = (unsigned)(jt0 - lo);
            vspan[nb] = (unsigned)(hi - lo);
            part = part || (on && !(jt0 >= lo && jt0 + 63 <= hi));
            off_row = off_row || !on;
          }
          // token scores take a max over every row of the tile, so there rows
          // that see nothing must hold -inf as well
          if (MODE != M_SPARSE_TOKEN)
            elem_mask = __ballot(part || (MODE == M_FULL_TILE && off_row)) != 0ull;
        }
        if (elem_mask) {
#pragma unroll
          for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
            for (int i4 = 0; i4 < 4; ++i4) {
              const int off = mb * 32 + 8 * i4 + 4 * hh;
              int4 ki = make_int4(0, 0, 0, 0);
              if (MODE == M_SPARSE_TOKEN) ki = *(const int4*)&kic[off];
#pragma unroll
              for (int e = 0; e < 4; ++e) {
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) {
                  bool ok;
                  if (MODE == M_SPARSE_TOKEN) {
                    const int kinf = e == 0 ? ki.x : (e == 1 ? ki.y : (e == 2 ? ki.z : ki.w));
                    const int j = kinf & 0x3fffffff;
                    const int ap = qpos[nb] + a.q_off;
                    ok = row_on[nb] && j <= ap && ((kinf >> 30) || (j > ap - a.window));
                  } else {
                    // key jt0 + off + e lies in [lo, hi]
                    ok = row_on[nb] && (vbase[nb] + (unsigned)(off + e)) <= vspan[nb];
                  }
                  if (!ok) s[mb][nb][4 * i4 + e] = kNegInf;
                }
              }
            }
          }
        }

        // token scores: per-key max over this workgroup's rows.  Register
        // x = 16 mb + i of lane (ln, hh) holds key mb*32 + 8(i/4) + 4hh + i%4
        // of row ln; colmax32 leaves the maxima of keys off .. off+3 in every
        // lane of a quad and the quad's first lane stores them.
        if (MODE == M_FULL_TILE) {
          float cm[32];
#pragma unroll
          for (int mb = 0; mb < 2; ++mb)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              float v = s[mb][0][i];
#pragma unroll
              for (int nb = 1; nb < NB; ++nb) v = fmax_nc(v, s[mb][nb][i]);
              cm[mb * 16 + i] = v;
            }
          const f32x4 m4 = colmax32(cm);
          const int off = (ln >> 4) * 32 + 8 * ((ln >> 2) & 3) + 4 * hh;
          if ((ln & 3) == 0) *(f32x4*)&red[(n & 1) * RS + wave * 64 + off] = m4;
        }

        // online softmax (base 2 on raw dot products) with a lazily updated
        // reference maximum: a row's reference moves only when the tile max
        // exceeds it by more than kLazyLog2 (probabilities then stay below
        // 2^kLazyLog2), so O and l are rescaled in few tiles.  The final
        // normalisation and the LSE use the same reference, so the result is
        // exact up to rounding.
        float alpha[NB];
        bool moved = false;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          float mt = kNegInf;
#pragma unroll
          for (int mb = 0; mb < 2; ++mb)
#pragma unroll
            for (int i = 0; i < 16; ++i) mt = fmaxf(mt, s[mb][nb][i]);
          mt = xor32_max(mt);
          if (!row_on[nb]) mt = kNegInf;
          if (MODE == M_FULL_BLOCK) {
            if (lane_scores) {
              // heads of a query are HC adjacent lanes: reduce them in-wave and
              // let the group's first lane store the block score
              float gm = mt;
              switch (HC) {
                case 2: gm = group_max<2>(mt); break;
                case 4: gm = group_max<4>(mt); break;
                case 8: gm = group_max<8>(mt); break;
                case 16: gm = group_max<16>(mt); break;
                case 32: gm = group_max<32>(mt); break;
                default: break;
              }
              if (hh == 0 && valid[nb] && (ln % HC) == 0)
                a.scores[(int64_t)g * a.sc_sg + (int64_t)b * a.sc_sb + (int64_t)qpos[nb] * a.sc_sr + n] =
                    gm * a.logit_scale;
            } else if (hh == 0) {
              red[(n & 1) * RS + wave * 32 * NB + nb * 32 + ln] = mt;
            }
          }
          // true when the reference is -inf and mt finite; false when both are -inf
          const bool need = mt > m_run[nb] + lazy_raw;
          const float mref = need ? mt : m_run[nb];
          alpha[nb] = need ? __builtin_amdgcn_exp2f((m_run[nb] - mref) * c2) : 1.f;
          moved = moved || need;
          m_run[nb] = mref;
          // rows that see nothing in this tile get probability 0 everywhere
          const float mc = !row_on[nb] ? __builtin_huge_valf() : ((mref == kNegInf) ? 0.f : mref * c2);
#pragma unroll
          for (int mb = 0; mb < 2; ++mb)
#pragma unroll
            for (int i = 0; i < 16; ++i) s[mb][nb][i] = __builtin_amdgcn_exp2f(fmaf(s[mb][nb][i], c2, -mc));
          // the row sum is taken over the fp32 probabilities, so the LSE is
          // the exact log-sum-exp up to fp32 rounding
          float ps = 0.f;
#pragma unroll
          for (int mb = 0; mb < 2; ++mb)
#pragma unroll
            for (int i = 0; i < 16; ++i) ps += s[mb][nb][i];
          l_run[nb] = fmaf(l_run[nb], alpha[nb], ps);
        }
        if (__ballot(moved) != 0ull) {
#pragma unroll
          for (int nb = 0; nb < NB; ++nb)
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
              for (int i = 0; i < 16; ++i) acc[nb][db][i] *= alpha[nb];
        }

        // O^T += V^T P^T  (M = D, N = rows, K = 64 keys); V^T fragments read one step ahead
        if constexpr (F32) {
          float vn = Vc[ln * VROW + 4 * hh];
#pragma unroll
          for (int st = 0; st < 32 * NDB; ++st) {
            const int kk = st / NDB, db = st % NDB;
            const int mb = kk >> 4, i = kk & 15;
            const float va = vn;
            if (st + 1 < 32 * NDB) {
              const int kk2 = (st + 1) / NDB, db2 = (st + 1) % NDB;
              const int key2 = (kk2 >> 4) * 32 + 8 * ((kk2 & 15) >> 2) + 4 * hh + (kk2 & 3);
              vn = Vc[(db2 * 32 + ln) * VROW + key2];
            }
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
              acc[nb][db] = __builtin_amdgcn_mfma_f32_32x32x2f32(va, s[mb][nb][i], acc[nb][db], 0, 0, 0);
          }
        } else {
          bf16x8 pf[4][NB];
#pragma unroll
          for (int kc = 0; kc < 4; ++kc) {
            const int mb = kc >> 1, i0 = 8 * (kc & 1);
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
              uint4 pk;
              pk.x = pack_bf16x2(s[mb][nb][i0 + 0], s[mb][nb][i0 + 1]);
              pk.y = pack_bf16x2(s[mb][nb][i0 + 2], s[mb][nb][i0 + 3]);
              pk.z = pack_bf16x2(s[mb][nb][i0 + 4], s[mb][nb][i0 + 5]);
              pk.w = pack_bf16x2(s[mb][nb][i0 + 6], s[mb][nb][i0 + 7]);
              pf[kc][nb] = as_bf16x8(pk);
            }
          }
#pragma unroll
          for (int db = 0; db < NDB; ++db) {
            if (db + 1 < NDB) {
#pragma unroll
              for (int kc = 0; kc < 4; ++kc) vf[db + 1][kc] = vfrag(db + 1, kc);
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int kc = 0; kc < 4; ++kc)
#pragma unroll
              for (int nb = 0; nb < NB; ++nb)
                acc[nb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(vf[db][kc]), pf[kc][nb], acc[nb][db], 0, 0, 0);
          }
        }
      }

      // stage tile n+1 into the other buffer, fetch tile n+2
      if (n + 1 < ntiles) stage_store((n + 1) & 1);
      if (n + 2 < ntiles) stage_load(n + 2, g);
      __syncthreads();
    }  // tile loop

    if (ntiles > 0) emit_scores(ntiles - 1);
    if (MODE == M_SPARSE_SWA && nsp == ntiles) finish_sparse_branch();

    // -inf for blocks / keys after the diagonal
    if (MODE == M_FULL_BLOCK) {
      float* sc = a.scores + (int64_t)g * a.sc_sg + (int64_t)b * a.sc_sb;
      const int c0 = ntiles, ncol = a.nblk - c0;
      if (ncol > 0)
        for (int e = tid; e < a.BQ * ncol; e += 256) {
          const int t = e / ncol, c = c0 + (e - t * ncol);
          if (q0 + t < a.Lq) sc[(int64_t)(q0 + t) * a.sc_sr + c] = kNegInf;
        }
    }

    // ---- epilogue ------------------------------------------------------------
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const float lsum = l_run[nb] + __shfl_xor(l_run[nb], 32);
      const bool live = m_run[nb] != kNegInf;
      const float inv = live ? a.v_scale / lsum : 0.f;
      const float lse_v = live ? (m_run[nb] * a.logit_scale + __logf(lsum)) : kNegInf;
      if (!valid[nb]) continue;
      const int64_t row_off_o = (int64_t)b * a.o_sb + (int64_t)qpos[nb] * a.o_st + (int64_t)head[nb] * a.o_sh;
      float gate = 1.f;
      bool sp_on = true;
      const float* osp = nullptr;
      // M_SWA_GATE without gate weights is the window branch alone (O and LSE)
      const bool gated = MODE == M_SPARSE_SWA || (MODE == M_SWA_GATE && a.gate_w != nullptr);
      if (gated) {
        // g = sigmoid(<q, w_h> + b_h): each lane holds half of the row's d values
        const float* w = a.gate_w + (int64_t)head[nb] * D;
        float z = 0.f;
        const QT* qr = qbase + (int64_t)qpos[nb] * a.q_st + (int64_t)head[nb] * a.q_sh;
#pragma unroll
        for (int c = 0; c < NQC; ++c) {
          if constexpr (F32) {
            z = fmaf(qr[2 * c + hh], w[2 * c + hh], z);
          } else {
            const uint4 qv = *(const uint4*)(qr + 16 * c + 8 * hh);
#pragma unroll
            for (int p = 0; p < 4; ++p) {
              const uint32_t wv = u4get(qv, p);
              z = fmaf(bf16_to_f32((uint16_t)(wv & 0xffffu)), w[16 * c + 8 * hh + 2 * p], z);
              z = fmaf(bf16_to_f32((uint16_t)(wv >> 16)), w[16 * c + 8 * hh + 2 * p + 1], z);
            }
          }
        }
        z += __shfl_xor(z, 32);
        if (a.gate_b) z += a.gate_b[head[nb]];
        gate = 1.f / (1.f + __expf(-z));
        if (MODE == M_SWA_GATE) {
          const float lsp = a.lse_sp[((int64_t)b * a.Hq + head[nb]) * a.Lq + qpos[nb]];
          sp_on = lsp != kNegInf;
          osp = a.o_sp + (int64_t)b * a.osp_sb + (int64_t)qpos[nb] * a.osp_st + (int64_t)head[nb] * a.osp_sh;
        } else {
          sp_on = sp_live[nb];
        }
      } else if (a.lse && hh == 0) {
        a.lse[((int64_t)b * a.Hq + head[nb]) * a.Lq + qpos[nb]] = lse_v;
      }
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          const int d = db * 32 + 8 * i4 + 4 * hh;
          float r[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) r[e] = acc[nb][db][4 * i4 + e] * inv;
          if (gated && sp_on) {
            float spv[4];
            if (MODE == M_SWA_GATE) {
              const float4 sp = *(const float4*)(osp + d);
              spv[0] = sp.x; spv[1] = sp.y; spv[2] = sp.z; spv[3] = sp.w;
            } else if (a.o_f32) {
              // the sparse branch this lane stored at the branch switch
              const float4 sp = *(const float4*)((const float*)a.o + row_off_o + d);
              spv[0] = sp.x; spv[1] = sp.y; spv[2] = sp.z; spv[3] = sp.w;
            } else {
              const uint2 sp = *(const uint2*)((const uint16_t*)a.o + row_off_o + d);
              spv[0] = bf16_to_f32((uint16_t)(sp.x & 0xffffu)); spv[1] = bf16_to_f32((uint16_t)(sp.x >> 16));
              spv[2] = bf16_to_f32((uint16_t)(sp.y & 0xffffu)); spv[3] = bf16_to_f32((uint16_t)(sp.y >> 16));
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) r[e] = gate * spv[e] + (1.f - gate) * r[e];
          }
          if (a.o_f32) {
            float4 out = {r[0], r[1], r[2], r[3]};
            *(float4*)((float*)a.o + row_off_o + d) = out;
          } else {
            uint2 out;
            out.x = pack_bf16x2(r[0], r[1]);
            out.y = pack_bf16x2(r[2], r[3]);
            *(uint2*)((uint16_t*)a.o + row_off_o + d) = out;
          }
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// per-mode launch (instantiated in one translation unit per mode)
// ---------------------------------------------------------------------------
// One 32-row MFMA block per wave (NB = 1): two workgroups per CU.  The engine
// is written for NB 32-row blocks per wave; NB = 2 (64 rows per wave) measured
// slower (one wave per SIMD, spills) and is not instantiated.
template <int MODE, typename QT, typename KT, int D>
static hipError_t launch_one(const AttnArgs& a, int grid, hipStream_t s) {
  if (a.nb != 1) return hipErrorInvalidValue;
  hipLaunchKernelGGL((attn_tile_kernel<MODE, QT, KT, D, 1>), dim3(grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

template <int MODE>
hipError_t launch_mode(int qt, int kt, int D, const AttnArgs& a, int grid, hipStream_t s) {
  if (qt == ET_F32 && kt == ET_F32) {
    if (D == 64) return launch_one<MODE, float, float, 64>(a, grid, s);
    if (D == 128) return launch_one<MODE, float, float, 128>(a, grid, s);
  } else if (qt == ET_BF16 && kt == ET_BF16) {
    if (D == 64) return launch_one<MODE, uint16_t, uint16_t, 64>(a, grid, s);
    if (D == 128) return launch_one<MODE, uint16_t, uint16_t, 128>(a, grid, s);
  } else if (qt == ET_BF16 && kt == ET_FP8) {
    if (D == 64) return launch_one<MODE, uint16_t, uint8_t, 64>(a, grid, s);
    if (D == 128) return launch_one<MODE, uint16_t, uint8_t, 128>(a, grid, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace hys
