// HySparse2 decode step kernels (gfx950): one new query per sequence against a
// long MQA KV cache stored as fp8 e4m3 (or bf16).
//
// The pages analyse decode at 1M tokens with an FP8 KV cache (airebao
// HySparse2 news, key-data table) and note that decoding keeps the whole
// cache, so memory bandwidth dominates (QbitAI HySparse article, background
// section).  The full layer therefore streams the cache once:
//
//   decode_kernel<full>   - split-K: every wave streams its own 64-key tiles
//                           through a private LDS slice (K as MFMA A fragments,
//                           V transposed), computes S^T = K q^T for all query
//                           heads at once (heads are the MFMA N dimension), and
//                           keeps an online-softmax partial.  The per-key max
//                           over heads is the token score, written directly.
//                           The 4 waves of a workgroup merge their partials in
//                           LDS, so one (m, l, O) partial per workgroup leaves.
//   decode_merge_kernel   - combines the partials in a fixed order (exact LSE
//                           rule, deterministic).
//   decode_kernel<sparse> - all sparse layers in one launch: each workgroup
//                           builds the layer-independent token list
//                           (selected tokens before the recent window, then the
//                           window itself) and gathers its share of the tiles.
#include "common.h"
#include "kernels.h"

namespace hys {

template <int SPARSE, typename KT, int D>
__global__ __launch_bounds__(256) void decode_kernel(const DecArgs a) {
  constexpr int KROW = D + 8;                 // bf16 LDS row stride of K
  constexpr int VROW = 68;                    // bf16 LDS row stride of V^T
  constexpr int WSLICE = 64 * KROW + D * VROW;
  constexpr int NDB = D / 32;
  constexpr int NQC = D / 16;
  constexpr int KUN = 64 * (D / 8);           // K units (8 elements) per tile
  constexpr int KU = KUN / 64;                // per lane
  constexpr int VUN = 16 * (D / 8);           // V units (4 keys x 8 d)
  constexpr int VU = VUN / 64;
  constexpr int TLMAX = 2048;
  static_assert(4 * WSLICE * 2 >= 4 * 64 * D * 4 + 2 * 4 * 64 * 4, "combine scratch must fit");

  __shared__ __attribute__((aligned(16))) uint16_t lds[4 * WSLICE];
  __shared__ int s_tlist[SPARSE ? TLMAX : 1];
  __shared__ int s_misc[8];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, hh = lane >> 5, ln = lane & 31;
  const int bid = blockIdx.x;
  const int s = bid % a.nsplit;
  const int rest = bid / a.nsplit;
  const int b = rest % a.B;
  const int layer = rest / a.B;
  const int n = a.lens[b];
  uint16_t* Kl = lds + wave * WSLICE;
  uint16_t* Vl = Kl + 64 * KROW;

  // ---- key list ------------------------------------------------------------
  int npre = 0, wstart = 0, nkeys = 0, ntiles_all = 0;
  if (!SPARSE) {
    nkeys = n;
    ntiles_all = (a.Nmax + 63) / 64;
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
      int before = carry;
      for (int w = 0; w < wave; ++w) before += s_misc[w];
      const int pos = before + __popcll(bal & ((1ull << lane) - 1ull));
      if (pre && pos < TLMAX) s_tlist[pos] = sv;
      carry += s_misc[0] + s_misc[1] + s_misc[2] + s_misc[3];
      __syncthreads();
    }
    npre = min(carry, TLMAX);
    nkeys = npre + (n - wstart);
    ntiles_all = (nkeys + 63) / 64;
  }
  const int ntiles_valid = (nkeys + 63) / 64;

  auto keyof = [&](int t, int x) -> int {     // key position of list slot 64t+x, or -1
    const int p = t * 64 + x;
    if (!SPARSE) return p < n ? p : -1;
    if (p < npre) return s_tlist[p];
    return p < nkeys ? wstart + (p - npre) : -1;
  };

  // ---- query fragments: heads are the 64 rows (2 N-blocks of 32) -----------
  const uint16_t* qb = (const uint16_t*)a.q[layer] + (int64_t)b * a.q_sb;
  bf16x8 qf[2][NQC];
  bool hvalid[2];
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    const int h = nb * 32 + ln;
    hvalid[nb] = h < a.Hq;
#pragma unroll
    for (int c = 0; c < NQC; ++c) {
      uint4 z = {0u, 0u, 0u, 0u};
      qf[nb][c] = as_bf16x8(hvalid[nb] ? *(const uint4*)(qb + (int64_t)h * a.q_sh + 16 * c + 8 * hh) : z);
    }
  }

  float m_run[2] = {kNegInf, kNegInf}, l_run[2] = {0.f, 0.f};
  f32x16 acc[2][NDB];
#pragma unroll
  for (int nb = 0; nb < 2; ++nb)
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[nb][db][i] = 0.f;

  const KT* kb = (const KT*)a.k + (int64_t)b * a.k_sb;
  const KT* vb = (const KT*)a.v + (int64_t)b * a.v_sb;
  Raw8<KT> kreg[KU];
  Raw8<KT> vreg[VU][4];

  auto stage_load = [&](int t) {
#pragma unroll
    for (int u = 0; u < KU; ++u) {
      const int unit = lane + 64 * u;
      const int key = unit / (D / 8), c8 = unit % (D / 8);
      const int j = keyof(t, key);
      kreg[u] = j >= 0 ? load8<KT>(kb + (int64_t)j * a.k_st + c8 * 8) : zero8<KT>();
    }
#pragma unroll
    for (int u = 0; u < VU; ++u) {
      const int unit = lane + 64 * u;
      const int kg = unit / (D / 8), dc = unit % (D / 8);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int j = keyof(t, kg * 4 + r);
        vreg[u][r] = j >= 0 ? load8<KT>(vb + (int64_t)j * a.v_st + dc * 8) : zero8<KT>();
      }
    }
  };
  auto stage_store = [&]() {
#pragma unroll
    for (int u = 0; u < KU; ++u) {
      const int unit = lane + 64 * u;
      const int key = unit / (D / 8), c8 = unit % (D / 8);
      *(uint4*)&Kl[key * KROW + c8 * 8] = to_ct(kreg[u]).a;
    }
#pragma unroll
    for (int u = 0; u < VU; ++u) {
      const int unit = lane + 64 * u;
      const int kg = unit / (D / 8), dc = unit % (D / 8);
      const uint4 r0 = to_ct(vreg[u][0]).a, r1 = to_ct(vreg[u][1]).a, r2 = to_ct(vreg[u][2]).a, r3 = to_ct(vreg[u][3]).a;
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const uint32_t w0 = u4get(r0, p), w1 = u4get(r1, p), w2 = u4get(r2, p), w3 = u4get(r3, p);
        uint2 e, o;
        e.x = __builtin_amdgcn_perm(w1, w0, 0x05040100u); e.y = __builtin_amdgcn_perm(w3, w2, 0x05040100u);
        o.x = __builtin_amdgcn_perm(w1, w0, 0x07060302u); o.y = __builtin_amdgcn_perm(w3, w2, 0x07060302u);
        *(uint2*)&Vl[(dc * 8 + 2 * p) * VROW + kg * 4] = e;
        *(uint2*)&Vl[(dc * 8 + 2 * p + 1) * VROW + kg * 4] = o;
      }
    }
  };

  const float c2 = a.scale_log2;
  const int gw = s * 4 + wave, gstride = a.nsplit * 4;
  int t = gw;
  if (t < ntiles_valid) stage_load(t);
  for (; t < ntiles_valid; t += gstride) {
    stage_store();
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    if (t + gstride < ntiles_valid) stage_load(t + gstride);

    f32x16 sacc[2][2];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int i = 0; i < 16; ++i) sacc[mb][nb][i] = 0.f;
#pragma unroll
    for (int c = 0; c < NQC; ++c)
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        const bf16x8 ka = as_bf16x8(*(const uint4*)&Kl[(mb * 32 + ln) * KROW + 16 * c + 8 * hh]);
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
          sacc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[nb][c], sacc[mb][nb], 0, 0, 0);
      }
    // mask: empty list slots and invalid heads
    const int rem = nkeys - t * 64;             // valid slots in this tile
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int off = mb * 32 + 8 * (i >> 2) + 4 * hh + (i & 3);
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
          if (off >= rem || !hvalid[nb]) sacc[mb][nb][i] = kNegInf;
      }
    if (!SPARSE) {
      // token score = max over heads; reduce-scatter so lane ln owns value index ln
      float cm[32];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int i = 0; i < 16; ++i) cm[mb * 16 + i] = fmaxf(sacc[mb][0][i], sacc[mb][1][i]);
#pragma unroll
      for (int st = 0; st < 5; ++st) {
        const int half = 16 >> st;
        const bool upper = (ln & half) != 0;
#pragma unroll
        for (int x = 0; x < half; ++x) {
          const float send = upper ? cm[x] : cm[x + half];
          const float keep = upper ? cm[x + half] : cm[x];
          cm[x] = fmaxf(keep, __shfl_xor(send, half));
        }
      }
      const int mb = ln >> 4, i = ln & 15;
      const int j = t * 64 + mb * 32 + 8 * (i >> 2) + 4 * hh + (i & 3);
      if (j < a.Nmax) a.scores[(int64_t)b * a.sc_sb + j] = (j < n) ? cm[0] * a.logit_scale : kNegInf;
    }
    // online softmax
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      float mt = kNegInf;
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int i = 0; i < 16; ++i) mt = fmaxf(mt, sacc[mb][nb][i]);
      mt = fmaxf(mt, __shfl_xor(mt, 32));
      const float mnew = fmaxf(m_run[nb], mt);
      const float muse = (mnew == kNegInf) ? 0.f : mnew;
      const float alpha = __builtin_amdgcn_exp2f((m_run[nb] - muse) * c2);
      m_run[nb] = mnew;
      const float mc = muse * c2;
      float ps = 0.f;
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float p = __builtin_amdgcn_exp2f(fmaf(sacc[mb][nb][i], c2, -mc));
          sacc[mb][nb][i] = p;
          ps += p;
        }
      l_run[nb] = fmaf(l_run[nb], alpha, ps);
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[nb][db][i] *= alpha;
    }
    // O^T += V^T P^T
#pragma unroll
    for (int kc = 0; kc < 4; ++kc) {
      const int mb = kc >> 1, i0 = 8 * (kc & 1);
      bf16x8 pf[2];
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        uint4 pk;
        pk.x = pack_bf16x2(sacc[mb][nb][i0 + 0], sacc[mb][nb][i0 + 1]);
        pk.y = pack_bf16x2(sacc[mb][nb][i0 + 2], sacc[mb][nb][i0 + 3]);
        pk.z = pack_bf16x2(sacc[mb][nb][i0 + 4], sacc[mb][nb][i0 + 5]);
        pk.w = pack_bf16x2(sacc[mb][nb][i0 + 6], sacc[mb][nb][i0 + 7]);
        pf[nb] = as_bf16x8(pk);
      }
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const uint16_t* vr = &Vl[(db * 32 + ln) * VROW + 16 * kc + 4 * hh];
        const uint2 lo = *(const uint2*)vr;
        const uint2 hi = *(const uint2*)(vr + 8);
        uint4 va; va.x = lo.x; va.y = lo.y; va.z = hi.x; va.w = hi.y;
        const bf16x8 vf = as_bf16x8(va);
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
          acc[nb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[nb], acc[nb][db], 0, 0, 0);
      }
    }
    __builtin_amdgcn_wave_barrier();
  }
  // tiles past the valid length: token scores are -inf
  if (!SPARSE) {
    for (int tt = t; tt < ntiles_all; tt += gstride) {   // t: this wave's first tile past the valid ones
      const int j = tt * 64 + lane;
      if (j < a.Nmax) a.scores[(int64_t)b * a.sc_sb + j] = kNegInf;
    }
  }

  // ---- merge the 4 waves' partials in LDS, emit one partial ----------------
  __syncthreads();
  float* Ow = (float*)lds;                       // [4][64 rows][D]
  float* Mw = Ow + 4 * 64 * D;                   // [4][64]
  float* Lw = Mw + 4 * 64;                       // [4][64]
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    const int row = nb * 32 + ln;
    const float lsum = l_run[nb] + __shfl_xor(l_run[nb], 32);
    if (hh == 0) { Mw[wave * 64 + row] = m_run[nb]; Lw[wave * 64 + row] = lsum; }
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const int d = db * 32 + 8 * i4 + 4 * hh;
        float4 v4 = {acc[nb][db][4 * i4], acc[nb][db][4 * i4 + 1], acc[nb][db][4 * i4 + 2], acc[nb][db][4 * i4 + 3]};
        *(float4*)&Ow[(wave * 64 + row) * D + d] = v4;
      }
  }
  __syncthreads();
  {
    const int row = tid >> 2, dq = (tid & 3) * (D / 4);
    if (row < a.Hq) {
      float m = kNegInf;
#pragma unroll
      for (int w = 0; w < 4; ++w) m = fmaxf(m, Mw[w * 64 + row]);
      float sc[4], l = 0.f;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float mw = Mw[w * 64 + row];
        sc[w] = (mw == kNegInf) ? 0.f : __builtin_amdgcn_exp2f((mw - m) * c2);
        l += Lw[w * 64 + row] * sc[w];
      }
      const int64_t pidx = ((int64_t)(layer * a.B + b) * a.nsplit + s) * a.Hq + row;
      float* po = a.part_o + pidx * D + dq;
      for (int d = 0; d < D / 4; d += 4) {
        float4 r = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const float4 x = *(const float4*)&Ow[(w * 64 + row) * D + dq + d];
          r.x += x.x * sc[w]; r.y += x.y * sc[w]; r.z += x.z * sc[w]; r.w += x.w * sc[w];
        }
        *(float4*)(po + d) = r;
      }
      if ((tid & 3) == 0) { a.part_ml[pidx * 2] = m; a.part_ml[pidx * 2 + 1] = l; }
    }
  }
}

// One workgroup per (layer, sequence, head); thread d combines the partials of
// output column d in split order.
template <int D>
__global__ __launch_bounds__(D) void decode_merge_kernel(const MergeArgs a) {
  const int bid = blockIdx.x;
  const int h = bid % a.Hq;
  const int b = (bid / a.Hq) % a.B;
  const int layer = bid / (a.Hq * a.B);
  const int d = threadIdx.x;
  const int64_t base = (int64_t)(layer * a.B + b) * a.nsplit;
  float m = kNegInf;
  for (int s = 0; s < a.nsplit; ++s) m = fmaxf(m, a.part_ml[((base + s) * a.Hq + h) * 2]);
  float l = 0.f, o = 0.f;
  if (m != kNegInf) {
    for (int s = 0; s < a.nsplit; ++s) {
      const int64_t p = (base + s) * a.Hq + h;
      const float ms = a.part_ml[p * 2];
      const float w = (ms == kNegInf) ? 0.f : __builtin_amdgcn_exp2f((ms - m) * a.scale_log2);
      l += a.part_ml[p * 2 + 1] * w;
      o += a.part_o[p * D + d] * w;
    }
  }
  const float out = (m != kNegInf) ? o / l * a.v_scale : 0.f;
  const int64_t off = (int64_t)b * a.o_sb + (int64_t)h * a.o_sh + d;
  if (a.o_f32) ((float*)a.o[layer])[off] = out;
  else ((uint16_t*)a.o[layer])[off] = f32_to_bf16(out);
  if (a.lse[layer] && d == 0)
    a.lse[layer][(int64_t)b * a.Hq + h] = (m != kNegInf) ? m * a.logit_scale + __logf(l) : kNegInf;
}

hipError_t launch_decode(int sparse, int kt, int D, const DecArgs& a, hipStream_t s) {
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

hipError_t launch_decode_merge(int D, const MergeArgs& a, hipStream_t s) {
  const unsigned grid = (unsigned)(a.nlayer * a.B * a.Hq);
  if (D == 128) hipLaunchKernelGGL(decode_merge_kernel<128>, dim3(grid), dim3(128), 0, s, a);
  else if (D == 64) hipLaunchKernelGGL(decode_merge_kernel<64>, dim3(grid), dim3(64), 0, s, a);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace hys
