// HySparse2 decode step kernels (gfx950): one new query per sequence against a
// long MQA KV cache stored as fp8 e4m3 (or bf16).
//
// The pages analyse decode at 1M tokens with an FP8 KV cache (airebao
// HySparse2 news, key-data table) and note that decoding keeps the whole
// cache, so memory bandwidth dominates (QbitAI HySparse article, background
// section).  The full layer therefore streams the cache once:
//
//   decode_kernel<full>   - split-K (bf16 caches, D = 64, and fp8 caches whose
//                           layout does not suit 16-byte LDS-direct loads; the
//                           fp8 D = 128 full layer otherwise runs the
//                           all-compute kernel of decode_split.hip): each
//                           workgroup takes a contiguous share
//                           of the 64-key tiles.  Two staging waves load fp8
//                           tiles several ahead and write them, as bf16 rows
//                           (K and V row-major), into a two-stage LDS ring;
//                           two compute waves (32 query heads each, the MFMA
//                           N dimension) take S^T = K q^T and O^T = V^T P^T
//                           from it with an online softmax, the V^T fragments
//                           by transposing LDS reads.  The per-key
//                           max over heads is the token score, written
//                           directly; each compute wave leaves one (m, l, O)
//                           partial per head.
//   decode_merge_kernel   - combines the partials in a fixed order (exact LSE
//                           rule, deterministic).
//   decode_kernel<sparse> - all sparse layers in one launch: each workgroup
//                           builds the layer-independent token list
//                           (selected tokens before the recent window, then the
//                           window itself) and gathers its share of the tiles.
#include "common.h"
#include "kernels.h"
#include "decode_split.h"
#include <type_traits>

namespace hys {

// f(integral_constant<int, I>) for I = 0 .. N-1, unrolled
template <int N, int I = 0, typename F>
__device__ __forceinline__ void dec_static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    dec_static_for<N, I + 1>(f);
  }
}

template <int SPARSE, typename KT, int D>
__global__ __launch_bounds__(256, 2) void decode_kernel(const DecArgs a) {
  // Workgroup = 4 waves.  Two compute: role w owns query heads
  // [32w, 32w+32) (one MFMA N-block) and both consume the same staged 64-key
  // tile, so every cache byte is read once per workgroup.  The other two
  // stage: they keep the loads of the next NSET tiles in flight in their own
  // registers and write each tile, converted to bf16 rows, into a two-stage
  // LDS ring one tile ahead of the compute waves, so these wait on LDS only,
  // never on memory latency.  One barrier per tile.
  //
  // LDS: K rows padded to KROW (read as MFMA A fragments, ds_read_b128); V
  // rows unpadded with the 16-byte chunks of key row r stored at chunk
  // c ^ vswz(r), read as V^T fragments by ds_read_b64_tr_b16 (within each
  // 16-lane slice, lane i receives element i of the four 4-element rows the
  // slice addresses: four consecutive keys of one d); the swizzle keeps
  // those reads free of bank conflicts.
  constexpr int KROW = D + 8;                 // bf16 LDS row stride of K
  constexpr int NDB = D / 32;
  constexpr int NQC = D / 16;
  constexpr int NST = 128;                    // staging threads
  constexpr int KU = 64 * (D / 8) / NST;      // K units (8 elements) per staging thread
  constexpr int VU = KU;                      // V units (8 elements of one key) per staging thread
  constexpr int NSET = sizeof(KT) == 1 ? 3 : 1;   // tiles of loads in flight
  constexpr int TLMAX = 2048;

  __shared__ __attribute__((aligned(16))) uint16_t Kl[2][64 * KROW];
  __shared__ __attribute__((aligned(16))) uint16_t Vl[2][64 * D];
  __shared__ __attribute__((aligned(16))) float red[2][2][64];
  __shared__ int s_tlist[SPARSE ? TLMAX : 1];
  __shared__ int s_misc[4];

  __shared__ int s_simd[4];
  // V row r: chunk c at c ^ vswz(r) (chosen by enumeration to keep the
  // transposing reads below free of conflicts on 32- and 64-bank LDS)
  auto vswz = [](int r) __attribute__((always_inline)) -> int {
    return D == 128 ? (5 * (r & 3)) & 15 : 2 * (r & 3);
  };
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, hh = lane >> 5, ln = lane & 31;
  const int bid = blockIdx.x;
  // Roles follow the SIMD a wave runs on.  The four waves of a workgroup sit
  // on four distinct SIMDs, and the two workgroups that share a CU are
  // dispatched in separate passes over the CUs; taking the compute waves on
  // SIMDs {0, 2} in one pass and {1, 3} in the other puts one compute wave on
  // every SIMD (fixed wave roles stacked both workgroups' compute waves on
  // one SIMD in every CU).  Any other placement keeps the fixed roles.
  // vw: role index, 0 and 1 compute (heads [32 vw, +32)), 2 and 3 stage.
  if (lane == 0) s_simd[wave] = (__builtin_amdgcn_s_getreg((31 << 11) | 4) >> 4) & 3;   // HW_REG_HW_ID.SIMD_ID
  __syncthreads();
  int vw = wave;
  if (((1 << s_simd[0]) | (1 << s_simd[1]) | (1 << s_simd[2]) | (1 << s_simd[3])) == 15) {
    const int my = s_simd[wave], par = (bid / a.ncu) & 1;
    vw = (((my + par) & 1) == 0 ? 0 : 2) + (my >> 1);
  }
  const bool stager = vw >= 2;
  const int st = (vw - 2) * 64 + lane;        // staging thread index (stager waves)
  const int s = bid % a.nsplit;
  const int rest = bid / a.nsplit;
  const int b = rest % a.B;
  const int layer = rest / a.B;
  const int n = a.lens[b];
  // full mode: layer l is the cache's KV head l (offsets 0 for one layer)
  float* const scr = SPARSE ? nullptr : a.scores + (int64_t)layer * a.sc_sl;

  // ---- key list ------------------------------------------------------------
  int npre = 0, wstart = 0, nkeys = 0;
  if (!SPARSE) {
    nkeys = n;
  } else {
    wstart = max(0, n - a.window);
    const int32_t* sel = a.idx + (int64_t)b * a.idx_sb;
    int carry = 0;
    for (int e0 = 0; e0 < a.topk; e0 += 256) {
      const int e = e0 + tid;
      const int sv = (e < a.topk) ? sel[e] : -1;
      const bool pre = sv >= 0 && sv < wstart;
      const unsigned long long bal = __ballot(pre);
      if (lane == 0) s_misc[wave] = __popcll(bal);
      __syncthreads();
      const int before = carry + (wave > 0 ? s_misc[0] : 0) + (wave > 1 ? s_misc[1] : 0) + (wave > 2 ? s_misc[2] : 0);
      const int pos = before + __popcll(bal & ((1ull << lane) - 1ull));
      if (pre && pos < TLMAX) s_tlist[pos] = sv;
      carry += s_misc[0] + s_misc[1] + s_misc[2] + s_misc[3];
      __syncthreads();
    }
    npre = min(carry, TLMAX);
    nkeys = npre + (n - wstart);
  }
  const int ntiles = (nkeys + 63) / 64;
  // this workgroup's contiguous share of the tiles
  const int per = (ntiles + a.nsplit - 1) / a.nsplit;
  const int t0 = s * per, t1 = min(ntiles, t0 + per);

  auto keyof = [&](int t, int x) -> int {     // key position of list slot 64t+x, or -1
    const int p = t * 64 + x;
    if (!SPARSE) return p < n ? p : -1;
    if (p < npre) return s_tlist[p];
    return p < nkeys ? wstart + (p - npre) : -1;
  };

  // ---- staging (roles 2, 3) ----------------------------------------------------
  // staging thread x, K or V unit u: key u*(NST/(D/8)) + x/(D/8), 8 elements
  // from x%(D/8)*8
  const KT* kb = (const KT*)a.k + (int64_t)b * a.k_sb + (SPARSE ? 0 : (int64_t)layer * a.k_sl);
  const KT* vb = (const KT*)a.v + (int64_t)b * a.v_sb + (SPARSE ? 0 : (int64_t)layer * a.v_sl);
  Raw8<KT> kreg[NSET][KU];
  Raw8<KT> vreg[NSET][VU];
  uint32_t kmask[NSET], vmask[NSET];
  bool sfull[NSET];
  const int koff0 = (st / (D / 8)) * (int)a.k_st + (st % (D / 8)) * 8;
  const int kstep = (NST / (D / 8)) * (int)a.k_st;
  const int voff0 = (st / (D / 8)) * (int)a.v_st + (st % (D / 8)) * 8;
  const int vstep = (NST / (D / 8)) * (int)a.v_st;

  auto stage_load = [&](auto set_tag, int t) __attribute__((always_inline)) {
    constexpr int S = decltype(set_tag)::value;
    // a contiguous tile of 64 valid keys: one uniform base, no masking
    sfull[S] = !SPARSE && t * 64 + 63 < n;
    if (sfull[S]) {
      const KT* kt = kb + (int64_t)t * 64 * a.k_st;
      const KT* vt = vb + (int64_t)t * 64 * a.v_st;
#pragma unroll
      for (int u = 0; u < KU; ++u) kreg[S][u] = load8<KT>(kt + koff0 + u * kstep);
#pragma unroll
      for (int u = 0; u < VU; ++u) vreg[S][u] = load8<KT>(vt + voff0 + u * vstep);
      return;
    }
    // loads are unconditional from a clamped in-bounds key (key 0); empty
    // slots are zeroed when staged (see keep_if)
    uint32_t km = 0u, vm = 0u;
#pragma unroll
    for (int u = 0; u < KU; ++u) {
      const int unit = u * NST + st;
      const int key = unit / (D / 8), c8 = unit % (D / 8);
      const int j = keyof(t, key);
      km |= (j >= 0 ? 1u : 0u) << u;
      kreg[S][u] = load8<KT>(kb + (int64_t)(j >= 0 ? j : 0) * a.k_st + c8 * 8);
    }
#pragma unroll
    for (int u = 0; u < VU; ++u) {
      const int unit = u * NST + st;
      const int key = unit / (D / 8), c8 = unit % (D / 8);
      const int j = keyof(t, key);
      vm |= (j >= 0 ? 1u : 0u) << u;
      vreg[S][u] = load8<KT>(vb + (int64_t)(j >= 0 ? j : 0) * a.v_st + c8 * 8);
    }
    kmask[S] = km; vmask[S] = vm;
  };
  auto stage_store = [&](auto set_tag, int stage) __attribute__((always_inline)) {
    constexpr int S = decltype(set_tag)::value;
    const bool full = sfull[S];
#pragma unroll
    for (int u = 0; u < KU; ++u) {
      const int unit = u * NST + st;
      const int key = unit / (D / 8), c8 = unit % (D / 8);
      if (!full) keep_if(kreg[S][u], (kmask[S] >> u) & 1u);
      *(uint4*)&Kl[stage][key * KROW + c8 * 8] = to_ct(kreg[S][u]).a;
    }
#pragma unroll
    for (int u = 0; u < VU; ++u) {
      const int unit = u * NST + st;
      const int key = unit / (D / 8), c8 = unit % (D / 8);
      if (!full) keep_if(vreg[S][u], (vmask[S] >> u) & 1u);
      *(uint4*)&Vl[stage][key * D + ((c8 ^ vswz(key)) * 8)] = to_ct(vreg[S][u]).a;
    }
  };

  // ---- query fragments (compute waves: this wave's 32 heads) -------------------
  const uint16_t* qb = (const uint16_t*)a.q[layer] + (int64_t)b * a.q_sb;
  const int head = vw * 32 + ln;
  const bool hvalid = !stager && head < a.Hq;
  bf16x8 qf[NQC];
#pragma unroll
  for (int c = 0; c < NQC; ++c) {
    const uint4 x = *(const uint4*)(qb + (int64_t)(hvalid ? head : 0) * a.q_sh + 16 * c + 8 * hh);
    const uint4 z = {0u, 0u, 0u, 0u};
    qf[c] = as_bf16x8(hvalid ? x : z);
  }

  // the lane's V^T read offset in a stage (d block 0, k-step 0)
  int vbase;
  {
    const int i = lane & 15, g = (lane >> 4) & 1;
    const int r = 4 * hh + (i >> 2), sv = vswz(r);
    const int x = 2 * g + ((i >> 1) & 1);            // chunk among the d block's four
    vbase = r * (2 * D) + 64 * (sv >> 2) + 16 * (x ^ (sv & 3)) + 8 * (i & 1);
  }

  float m_run = kNegInf, l_run = 0.f;
  f32x16 acc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[db][i] = 0.f;

  // token scores of tile t: max over the two compute waves' per-key maxima
  auto emit_scores = [&](int t) {
    if (!SPARSE && vw == 0) {
      const int j = t * 64 + lane;
      const float v = fmaxf(red[t & 1][0][lane], red[t & 1][1][lane]);
      if (j < a.Nmax) scr[(int64_t)b * a.sc_sb + j] = (j < n) ? v * a.logit_scale : kNegInf;
    }
  };

  const float c2 = a.scale_log2;
  const float lazy_raw = kLazyLog2 / c2;      // the reference slack in raw dot-product units
  // one tile of attention for this compute wave, from LDS stage t & 1
  auto compute = [&](int t) __attribute__((always_inline)) {
    const uint16_t* Kc = Kl[t & 1];
    const uint16_t* Vc = Vl[t & 1];
    // S^T = K q^T: 64 keys (2 M-blocks) x this wave's 32 heads; K fragments
    // are read two k-steps ahead of their MFMAs (pinned: the scheduler would
    // otherwise sink each read next to its MFMA and expose the LDS latency)
    f32x16 sacc[2];
    const f32x16 zero16 = {};
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
      __builtin_amdgcn_sched_barrier(0);
      sacc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(kf[c][0]), qf[c], c == 0 ? zero16 : sacc[0], 0, 0, 0);
      sacc[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(kf[c][1]), qf[c], c == 0 ? zero16 : sacc[1], 0, 0, 0);
    }
    // V^T fragments (A operand of O^T): the first d block is read now, under
    // the softmax; later blocks one d block ahead of their MFMAs
    // k-step kc of d block db, lane (slice g = lane/16, i = lane%16): keys
    // 16kc + 4hh + (0..3) (lo) and 16kc + 8 + 4hh + (0..3) (hi) at
    // d = 32db + 16(g%2) + i.  The slice addresses rows 4hh + i/4 (+16kc, +8)
    // at d = 32db + 16(g%2) + 4(i%4); vswz only flips the d-block bits and
    // those below, so the swizzled offset is the lane's base XOR 64db.
    auto vfrag = [&](int db, int kc) __attribute__((always_inline)) {
      typedef short v4i16 __attribute__((ext_vector_type(4)));
      typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
      const char* vr = (const char*)Vc + (vbase ^ (64 * db)) + (16 * kc) * (2 * D);
      const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)vr);
      const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(vr + 8 * (2 * D)));
      const uint2 l2 = __builtin_bit_cast(uint2, lo), h2 = __builtin_bit_cast(uint2, hi);
      uint4 va; va.x = l2.x; va.y = l2.y; va.z = h2.x; va.w = h2.y;
      return va;
    };
    uint4 vf[2][4];
#pragma unroll
    for (int kc = 0; kc < 4; ++kc) vf[0][kc] = vfrag(0, kc);
    __builtin_amdgcn_sched_barrier(0);
    // mask empty list slots and padding heads
    const int rem = nkeys - t * 64;
    if (rem < 64 || !hvalid) {
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int off = mb * 32 + 8 * (i >> 2) + 4 * hh + (i & 3);
          if (off >= rem || !hvalid) sacc[mb][i] = kNegInf;
        }
    }
    if (!SPARSE) {
      // per-key max over this wave's heads, reduced in registers: every lane
      // of a quad ends with the maxima of keys off .. off+3
      float cm[32];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int i = 0; i < 16; ++i) cm[mb * 16 + i] = sacc[mb][i];
      const f32x4 m4 = colmax32(cm);
      const int off = (ln >> 4) * 32 + 8 * ((ln >> 2) & 3) + 4 * hh;
      if ((ln & 3) == 0) *(f32x4*)&red[t & 1][vw][off] = m4;
    }
    // online softmax (base 2) with a lazily moved reference maximum: a
    // head's reference moves only when the tile max exceeds it by more than
    // kLazyLog2 (so probabilities stay below 2^kLazyLog2 and O is rescaled in
    // few tiles); O, l and the partial's m all use that reference, so the
    // merged result is exact up to rounding
    float mt = kNegInf;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int i = 0; i < 16; ++i) mt = fmaxf(mt, sacc[mb][i]);
    mt = xor32_max(mt);
    // true when the reference is -inf and mt finite; false when both are -inf
    const bool moved = mt > m_run + lazy_raw;
    const float mref = moved ? mt : m_run;
    const float alpha = moved ? __builtin_amdgcn_exp2f((m_run - mref) * c2) : 1.f;
    m_run = mref;
    const float mc = (mref == kNegInf) ? 0.f : mref * c2;
    float ps = 0.f;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float p = __builtin_amdgcn_exp2f(fmaf(sacc[mb][i], c2, -mc));
        sacc[mb][i] = p;
        ps += p;
      }
    l_run = fmaf(l_run, alpha, ps);
    if (__ballot(moved) != 0ull) {
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[db][i] *= alpha;
    }
    // O^T += V^T P^T, V^T fragments read one step ahead
    bf16x8 pf[4];
#pragma unroll
    for (int kc = 0; kc < 4; ++kc) {
      const int mb = kc >> 1, i0 = 8 * (kc & 1);
      uint4 pk;
      pk.x = pack_bf16x2(sacc[mb][i0 + 0], sacc[mb][i0 + 1]);
      pk.y = pack_bf16x2(sacc[mb][i0 + 2], sacc[mb][i0 + 3]);
      pk.z = pack_bf16x2(sacc[mb][i0 + 4], sacc[mb][i0 + 5]);
      pk.w = pack_bf16x2(sacc[mb][i0 + 6], sacc[mb][i0 + 7]);
      pf[kc] = as_bf16x8(pk);
    }
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      if (db + 1 < NDB) {
#pragma unroll
        for (int kc = 0; kc < 4; ++kc) vf[(db + 1) & 1][kc] = vfrag(db + 1, kc);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int kc = 0; kc < 4; ++kc)
        acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(vf[db & 1][kc]), pf[kc], acc[db], 0, 0, 0);
    }
  };

  // ---- tile pipeline: iteration i stages tile t0 + i (staging waves) while the
  // compute waves take tile t0 + i - 1; the stager's loads run NSET tiles
  // ahead.  The two roles run separate loops with the same barrier count, so
  // neither keeps the other's registers live.
  const int niter = (t1 > t0) ? (t1 - t0 + 1) : 0;
  if (stager) {
    dec_static_for<NSET>([&](auto set_tag) __attribute__((always_inline)) {
      constexpr int S = decltype(set_tag)::value;
      if (t0 + S < t1) stage_load(set_tag, t0 + S);
    });
    auto step = [&](int i, auto set_tag) __attribute__((always_inline)) {
      const int t = t0 + i;
      if (t < t1) {
        stage_store(set_tag, t & 1);
        if (t + NSET < t1) stage_load(set_tag, t + NSET);
      }
      __syncthreads();
    };
    for (int i = 0; i < niter; i += NSET) {
      dec_static_for<NSET>([&](auto set_tag) __attribute__((always_inline)) {
        constexpr int S = decltype(set_tag)::value;
        if (i + S < niter) step(i + S, set_tag);
      });
    }
  } else {
    for (int i = 0; i < niter; ++i) {
      const int t = t0 + i;
      if (i >= 2) emit_scores(t - 2);
      if (i >= 1) compute(t - 1);
      __syncthreads();
    }
  }
  if (t0 < t1) emit_scores(t1 - 1);
  // keys past the valid length: token scores are -inf (the workgroups of the
  // last split cover the tail of the score row)
  if (!SPARSE && s == a.nsplit - 1) {
    for (int j = ntiles * 64 + tid; j < a.Nmax; j += 256) scr[(int64_t)b * a.sc_sb + j] = kNegInf;
  }

  // ---- this wave's partial (m, l, unnormalised O) ------------------------------
  if (hvalid) {
    const float lsum = l_run + __shfl_xor(l_run, 32);
    const int64_t pidx = ((int64_t)(layer * a.B + b) * a.nsplit + s) * a.Hq + head;
    float* po = a.part_o + pidx * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const int d = db * 32 + 8 * i4 + 4 * hh;
        const float4 v4 = {acc[db][4 * i4], acc[db][4 * i4 + 1], acc[db][4 * i4 + 2], acc[db][4 * i4 + 3]};
        *(float4*)(po + d) = v4;
      }
    if (hh == 0) { a.part_ml[pidx * 2] = m_run; a.part_ml[pidx * 2 + 1] = lsum; }
  }
}

// One workgroup per (layer, sequence, head), in two passes.  First the
// workgroup takes the maximum M of the partials' reference maxima.  Then
// thread (g, q) sums the partials s = g, g + NG, g + 2 NG, ... of output
// columns [4q, 4q+4), each weighted by exp2((m_s - M) c) (the exact LSE
// rule with a common reference, so the sum has no serial dependence and the
// loads of many partials are in flight together), and the NG group sums are
// added in group order in LDS, so the result does not depend on scheduling.
template <int D>
__device__ __forceinline__ void decode_merge_one(const MergeArgs& a, int bid) {
  constexpr int NQ = D / 4;          // float4 column groups
  constexpr int NG = 256 / NQ;       // split groups
  __shared__ float sl[NG], smax[4];
  __shared__ float4 so[NG][NQ];
  const int h = bid % a.Hq;
  const int b = (bid / a.Hq) % a.B;
  const int layer = bid / (a.Hq * a.B);
  const int tid = threadIdx.x;
  const int q = tid % NQ, g = tid / NQ;
  const int64_t base = (int64_t)(layer * a.B + b) * a.nsplit;
  const float c2 = a.scale_log2;
  // pass 1: M = max over the splits' m
  float mx = kNegInf;
  for (int s = tid; s < a.nsplit; s += 256) mx = fmaxf(mx, a.part_ml[((base + s) * a.Hq + h) * 2]);
  mx = wave_max(mx);
  if ((tid & 63) == 0) smax[tid >> 6] = mx;
  __syncthreads();
  const float M = fmaxf(fmaxf(smax[0], smax[1]), fmaxf(smax[2], smax[3]));
  // pass 2: weighted sums (empty partials have m = -inf and weight 0)
  float l = 0.f;
  float4 o = {0.f, 0.f, 0.f, 0.f};
  if (M != kNegInf) {
#pragma unroll 4
    for (int s = g; s < a.nsplit; s += NG) {
      const int64_t p = (base + s) * a.Hq + h;
      const float ms = a.part_ml[p * 2], ls = a.part_ml[p * 2 + 1];
      const float4 os = *(const float4*)(a.part_o + p * D + 4 * q);
      const float w = ms == kNegInf ? 0.f : __builtin_amdgcn_exp2f((ms - M) * c2);
      l = fmaf(ls, w, l);
      o.x = fmaf(os.x, w, o.x); o.y = fmaf(os.y, w, o.y);
      o.z = fmaf(os.z, w, o.z); o.w = fmaf(os.w, w, o.w);
    }
  }
  if (q == 0) sl[g] = l;
  so[g][q] = o;
  __syncthreads();
  if (g == 0) {
    float L = 0.f;
    float4 O = {0.f, 0.f, 0.f, 0.f};
    for (int x = 0; x < NG; ++x) {
      L += sl[x];
      const float4 v = so[x][q];
      O.x += v.x; O.y += v.y; O.z += v.z; O.w += v.w;
    }
    const float inv = (M != kNegInf) ? a.v_scale / L : 0.f;
    const int64_t off = (int64_t)b * a.o_sb + (int64_t)h * a.o_sh + 4 * q;
    if (a.o_f32) {
      const float4 r = {O.x * inv, O.y * inv, O.z * inv, O.w * inv};
      *(float4*)((float*)a.o[layer] + off) = r;
    } else {
      uint2 r;
      r.x = pack_bf16x2(O.x * inv, O.y * inv);
      r.y = pack_bf16x2(O.z * inv, O.w * inv);
      *(uint2*)((uint16_t*)a.o[layer] + off) = r;
    }
    if (a.lse[layer] && q == 0)
      a.lse[layer][(int64_t)b * a.Hq + h] = (M != kNegInf) ? M * a.logit_scale + __logf(L) : kNegInf;
  }
}

template <int D>
__global__ __launch_bounds__(256) void decode_merge_kernel(const MergeArgs a) {
  decode_merge_one<D>(a, blockIdx.x);
}

// two merges in one launch (the full layer's and the sparse layers')
template <int D>
__global__ __launch_bounds__(256) void decode_merge2_kernel(const MergeArgs a, const MergeArgs b) {
  const int na = a.nlayer * a.B * a.Hq;
  if ((int)blockIdx.x < na) decode_merge_one<D>(a, blockIdx.x);
  else decode_merge_one<D>(b, blockIdx.x - na);
}

hipError_t launch_decode(int sparse, int kt, int D, const DecArgs& a, hipStream_t s) {
  if (!sparse && kt == ET_FP8 && decode_split_fp8_supported(D, a)) return launch_decode_split_fp8(a, s);
  // (the split kernel clears a.zero itself; the other paths clear it first)
  if (!sparse && a.zero) {
    hipError_t e = launch_fill_i32(a.zero, 0, a.zero_n, s);
    if (e != hipSuccess) return e;
  }
  const unsigned grid = (unsigned)(a.nlayer * a.B * a.nsplit);
#define HYS_DEC(SP, KT, DD) hipLaunchKernelGGL((decode_kernel<SP, KT, DD>), dim3(grid), dim3(256), 0, s, a)
  if (kt == ET_FP8) {
    if (D == 128) { if (sparse) HYS_DEC(1, uint8_t, 128); else HYS_DEC(0, uint8_t, 128); }
    else if (D == 64) { if (sparse) HYS_DEC(1, uint8_t, 64); else HYS_DEC(0, uint8_t, 64); }
    else return hipErrorInvalidValue;
  } else if (kt == ET_BF16) {
    if (D == 128) { if (sparse) HYS_DEC(1, uint16_t, 128); else HYS_DEC(0, uint16_t, 128); }
    else if (D == 64) { if (sparse) HYS_DEC(1, uint16_t, 64); else HYS_DEC(0, uint16_t, 64); }
    else return hipErrorInvalidValue;
  } else {
    return hipErrorInvalidValue;
  }
#undef HYS_DEC
  return hipGetLastError();
}

hipError_t launch_decode_merge2(int D, const MergeArgs& a, const MergeArgs& b, hipStream_t s) {
  const unsigned grid = (unsigned)(a.nlayer * a.B * a.Hq + b.nlayer * b.B * b.Hq);
  if (D == 128) hipLaunchKernelGGL(decode_merge2_kernel<128>, dim3(grid), dim3(256), 0, s, a, b);
  else if (D == 64) hipLaunchKernelGGL(decode_merge2_kernel<64>, dim3(grid), dim3(256), 0, s, a, b);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_decode_merge(int D, const MergeArgs& a, hipStream_t s) {
  const unsigned grid = (unsigned)(a.nlayer * a.B * a.Hq);
  if (D == 128) hipLaunchKernelGGL(decode_merge_kernel<128>, dim3(grid), dim3(256), 0, s, a);
  else if (D == 64) hipLaunchKernelGGL(decode_merge_kernel<64>, dim3(grid), dim3(256), 0, s, a);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace hys
