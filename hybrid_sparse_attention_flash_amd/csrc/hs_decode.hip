// HySparse (block-level) decode step kernels (gfx950): one new query per
// sequence against a bf16 GQA cache.  The full layer runs on the split-K
// decode kernel, one launch per KV head with that head's query group; these
// kernels turn its per-KV-head token scores into block scores and run every
// sparse layer.
//
// HySparse's hybrid block (QbitAI HySparse article, method section; TechWalker
// write-up): the full layer's kernel emits block-level maxima of its logits
// (64-token blocks), a top-k picks the blocks, and each sparse layer fuses a
// block-sparse branch over the shared cache with a sliding-window branch over
// its own window K/V by a sigmoid gate.  At decode the window K/V of a layer
// is a ring of W slots, token t in slot t mod W; the step appends the new
// token into slot (n-1) mod W and the window covers tokens [max(0, n-W), n-1].
//
//   hs_block_max_kernel      - block score M[b, c] = max over the KV heads'
//                              token scores of block c (one wave per block)
//   hs_decode_sparse_kernel  - per (layer, sequence, KV head, group of up to
//                              8 of its query heads), ceil(topk / 4) + 1
//                              workgroups: each of the first takes 4 selected
//                              blocks, one per wave, the last the window (and
//                              appends the new token to the ring); 64-key
//                              chunks with lane = key for the logits and the
//                              online softmax and lane = head dim for P V,
//                              the waves merged in LDS, and each workgroup's
//                              (max, sum, O) written per head
//   hs_decode_gate_kernel    - one wave per (layer, sequence, query head):
//                              merges the selected-block partials, then the
//                              gate with the window branch
#include "common.h"
#include "kernels.h"

namespace hys {

__global__ __launch_bounds__(256) void hs_block_max_kernel(const float* __restrict__ ts, int nparts,
                                                          int64_t part_stride, int B, int Nmax, int nblk,
                                                          float* __restrict__ out) {
  const int w = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (w >= B * nblk) return;
  const int b = w / nblk, c = w - b * nblk;
  const int j = c * 64 + lane;
  float m = kNegInf;
  if (j < Nmax)
    for (int p = 0; p < nparts; ++p) m = fmaxf(m, ts[p * part_stride + (int64_t)b * Nmax + j]);
  m = wave_max(m);
  if (lane == 0) out[(int64_t)b * nblk + c] = m;
}

hipError_t launch_hs_block_max(const float* ts, int nparts, int64_t part_stride, int B, int Nmax, int nblk,
                               float* out, hipStream_t s) {
  const int64_t waves = (int64_t)B * nblk;
  if (waves == 0) return hipSuccess;
  hipLaunchKernelGGL(hs_block_max_kernel, dim3((unsigned)((waves + 3) / 4)), dim3(256), 0, s, ts, nparts,
                     part_stride, B, Nmax, nblk, out);
  return hipGetLastError();
}

namespace {
constexpr int kHsGmax = 8;    // query heads per workgroup
constexpr int kHsKmax = 64;   // selected blocks
// native vectors (register arrays of HIP's uint4 wrapper struct end up in scratch)
typedef unsigned int hs_u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int hs_u32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ bf16x8 hs_frag(hs_u32x4 v) { return __builtin_bit_cast(bf16x8, v); }
__device__ __forceinline__ hs_u32x4 hs_pack8(const float* x) {
  return hs_u32x4{pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]), pack_bf16x2(x[4], x[5]), pack_bf16x2(x[6], x[7])};
}
}  // namespace

// GQ: query heads per workgroup (a KV head's a.G query heads are split into
// a.G / GQ sub-groups, one workgroup each).  Per 64-key chunk a wave runs
//   S^T = K Q^T    v_mfma_f32_32x32x16_bf16, A = 32 key rows (loaded straight
//                  into operand layout), B = the group's queries (columns
//                  >= GQ zero), two 32-key tiles;
//   softmax        per head = per lane column, the two half-waves combined;
//   O += P V       A = P as it leaves the S MFMA (lane = head, keys in the
//                  C-layout order, read by V in the same permuted order),
//                  B = V^T staged per wave through LDS, 32 keys at a time.
template <int D, int GQ>
__global__ __launch_bounds__(256) void hs_decode_sparse_kernel(const HsDecArgs a) {
  constexpr int NC = D / 16;                 // k-steps of S
  constexpr int NT = D / 32;                 // 32-wide d tiles of O
  constexpr int VTS = 36;                    // V^T row stride: 32 keys + 4 (conflict-free pair stores)
  __shared__ __attribute__((aligned(16))) uint32_t qs[kHsGmax][D / 2];   // bf16 pairs
  __shared__ __attribute__((aligned(16))) uint16_t vt[4][D * VTS];
  __shared__ float wm[4][kHsGmax], wl[4][kHsGmax];
  __shared__ __attribute__((aligned(16))) float wo[4][kHsGmax][D];
  __shared__ float alpha_s[4][32];
  __shared__ int sel[kHsKmax];

  // wave index as a wave-uniform value, so chunk and row addresses stay scalar
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ln = lane & 31, hh = lane >> 5;
  const int nsub = a.G / GQ;
  const int split = blockIdx.x % a.nsplit;    // 0..nsplit-2: selected blocks 4 split.., nsplit-1: window
  const int wg = blockIdx.x / a.nsplit;
  const bool win = split == a.nsplit - 1;
  const int sg = wg % nsub;                   // head sub-group
  const int g = (wg / nsub) % a.Hkv;
  const int rest = wg / (nsub * a.Hkv);
  const int b = rest % a.B;
  const int layer = rest / a.B;
  const int n = a.lens[b];
  const int h0 = g * a.G + sg * GQ;           // first query head of this workgroup
  const int W = a.W;

  // ---- append the new token's window K/V to the ring (slot (n-1) mod W held
  // token n-1-W, which is outside this step's window)
  {
    const int slot = (n - 1) % W;
    constexpr int U = D / 8;                 // 16-byte units per row
    if (win && sg == 0 && tid < 2 * U) {
      const bool isv = tid >= U;
      const int u = isv ? tid - U : tid;
      const uint16_t* src = (isv ? a.vnew[layer] : a.knew[layer]) + (int64_t)b * a.n_sb + (int64_t)g * a.n_sh;
      uint16_t* dst = (isv ? a.vring[layer] : a.kring[layer]) + (int64_t)b * a.r_sb + (int64_t)slot * a.r_st +
                      (int64_t)g * a.r_sh;
      *(uint4*)(dst + 8 * u) = *(const uint4*)(src + 8 * u);
    }
  }
  // ---- the group's queries and the selected blocks
  const uint16_t* qb = a.q[layer] + (int64_t)b * a.q_sb;
  for (int i = tid; i < kHsGmax * (D / 2); i += 256) {
    const int h = i / (D / 2), d2 = i - h * (D / 2);
    qs[h][d2] = h < GQ ? *(const uint32_t*)(qb + (int64_t)(h0 + h) * a.q_sh + 2 * d2) : 0u;
  }
  if (tid < kHsKmax) sel[tid] = tid < a.topk ? a.idx[(int64_t)b * a.idx_sb + tid] : -1;
  __syncthreads();

  // queries as B operand: lane (ln, hh) holds head ln, d = 16c + 8hh + [0, 8) (zero past GQ)
  hs_u32x4 qf[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c)
    qf[c] = ln < GQ ? *(const hs_u32x4*)&qs[ln][8 * c + 4 * hh] : hs_u32x4{0u, 0u, 0u, 0u};

  const uint16_t* kc = a.k + (int64_t)b * a.k_sb + (int64_t)g * a.k_sh;
  const uint16_t* vc = a.v + (int64_t)b * a.v_sb + (int64_t)g * a.v_sh;
  const uint16_t* kr = a.kring[layer] + (int64_t)b * a.r_sb + (int64_t)g * a.r_sh;
  const uint16_t* vr = a.vring[layer] + (int64_t)b * a.r_sb + (int64_t)g * a.r_sh;
  const uint16_t* kn = a.knew[layer] + (int64_t)b * a.n_sb + (int64_t)g * a.n_sh;
  const uint16_t* vn = a.vnew[layer] + (int64_t)b * a.n_sb + (int64_t)g * a.n_sh;
  const int wstart = max(0, n - W);
  const float c2 = a.scale_log2;

  // br 0: the selected blocks of the shared cache (one chunk per block, this
  // workgroup's four); br 1: the window (chunks of 64 positions from wstart)
  const int br = win ? 1 : 0;
  const int c0 = win ? 0 : 4 * split;
  const int nchunk = win ? (n - wstart + 63) / 64 : min(a.topk, c0 + 4);
  float m = kNegInf, l = 0.f;                // softmax state of head ln (both half-waves)
  f32x16 o[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[t][i] = 0.f;
  uint16_t* vtw = vt[wave];

  for (int c = c0 + wave; c < nchunk; c += 4) {
    const int blk = br == 0 ? __builtin_amdgcn_readfirstlane(sel[c]) : 0;   // uniform: scalar row addresses
    // position x = 0..63 of the chunk: row pointers and validity
    auto row = [&](int x, bool isv, bool& valid) -> const uint16_t* {
      if (br == 0) {
        const int j = blk * 64 + x;
        valid = blk >= 0 && j < n;
        return (isv ? vc : kc) + (int64_t)(valid ? j : 0) * (isv ? a.v_st : a.k_st);
      }
      const int t = wstart + c * 64 + x;
      valid = t < n;
      if (t == n - 1) return isv ? vn : kn;
      return (isv ? vr : kr) + (int64_t)((valid ? t : 0) % W) * a.r_st;
    };
    // K rows as A operands (key 32kt + ln, d = 16c + 8hh + [0, 8)) and the V
    // rows this lane stages (key pairs 2(ln % 16) + {0, 1} of each 32-key tile,
    // 16-byte chunks ln / 16 + 4u), all loads issued before use
    hs_u32x4 kf[2][NC];
    hs_u32x4 vraw[2][NT][2];
    bool kval[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      const uint16_t* kp = row(32 * kt + ln, false, kval[kt]);
#pragma unroll
      for (int cc = 0; cc < NC; ++cc) kf[kt][cc] = *(const hs_u32x4*)(kp + 16 * cc + 8 * hh);
    }
    const int vkp = lane & 15, vch = lane >> 4;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int u = 0; u < NT; ++u)
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          bool vv;
          const uint16_t* vp = row(32 * kt + 2 * vkp + e, true, vv);
          vraw[kt][u][e] = *(const hs_u32x4*)(vp + 8 * (vch + 4 * u));
        }
    // S^T per 32-key tile: lane (ln, hh) holds head ln, keys 32kt + 8(i/4) + 4hh + i%4
    f32x16 s[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
      for (int i = 0; i < 16; ++i) s[kt][i] = 0.f;
#pragma unroll
      for (int cc = 0; cc < NC; ++cc)
        s[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(hs_frag(kf[kt][cc]), hs_frag(qf[cc]), s[kt], 0, 0, 0);
    }
    // online softmax of head ln over the chunk (base 2); invalid keys are -inf
    float cmax = kNegInf;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int x = 32 * kt + 8 * (i >> 2) + 4 * hh + (i & 3);
        const bool ok = br == 0 ? (blk >= 0 && blk * 64 + x < n) : (wstart + c * 64 + x < n);
        s[kt][i] = ok ? s[kt][i] * c2 : kNegInf;
        cmax = fmaxf(cmax, s[kt][i]);
      }
    cmax = fmaxf(cmax, __shfl_xor(cmax, 32));
    const float mn = fmaxf(m, cmax);
    const float alpha = mn == kNegInf ? 1.f : exp2f(m - mn);
    float psum = 0.f;
    float p[2][16];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        p[kt][i] = s[kt][i] == kNegInf ? 0.f : exp2f(s[kt][i] - mn);
        psum += p[kt][i];
      }
    psum += __shfl_xor(psum, 32);
    l = l * alpha + psum;
    m = mn;
    // rescale O: its rows are heads 8(i/4) + 4hh + i%4, whose factors lane ln = head published
    if (hh == 0) alpha_s[wave][ln] = alpha;
    __asm__ volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float f = alpha_s[wave][8 * (i >> 2) + 4 * hh + (i & 3)];
#pragma unroll
      for (int t = 0; t < NT; ++t) o[t][i] *= f;
    }
    // O += P V, one 32-key tile at a time through this wave's V^T buffer
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      __asm__ volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // the previous tile's V^T reads are done
#pragma unroll
      for (int u = 0; u < NT; ++u) {
        const hs_u32x4 v0 = vraw[kt][u][0], v1 = vraw[kt][u][1];
        const int dch = vch + 4 * u;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint32_t x0 = v0[e >> 1], x1 = v1[e >> 1];
          const uint32_t wv = (e & 1) ? ((x0 >> 16) | (x1 & 0xffff0000u)) : ((x0 & 0xffffu) | (x1 << 16));
          *(uint32_t*)&vtw[(8 * dch + e) * VTS + 2 * vkp] = wv;
        }
      }
      __asm__ volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      const hs_u32x4 pa0 = hs_pack8(&p[kt][0]), pa1 = hs_pack8(&p[kt][8]);
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const uint16_t* tv = &vtw[(32 * t + ln) * VTS + 4 * hh];
        const hs_u32x4 b0 = {((const hs_u32x2*)tv)[0].x, ((const hs_u32x2*)tv)[0].y,
                             ((const hs_u32x2*)(tv + 8))[0].x, ((const hs_u32x2*)(tv + 8))[0].y};
        const hs_u32x4 b1 = {((const hs_u32x2*)(tv + 16))[0].x, ((const hs_u32x2*)(tv + 16))[0].y,
                             ((const hs_u32x2*)(tv + 24))[0].x, ((const hs_u32x2*)(tv + 24))[0].y};
        o[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(hs_frag(pa0), hs_frag(b0), o[t], 0, 0, 0);
        o[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(hs_frag(pa1), hs_frag(b1), o[t], 0, 0, 0);
      }
    }
  }
  // this wave's (max, sum, O) per head: O in C layout, lane (ln, hh) holds d =
  // 32t + ln of heads 8(i/4) + 4hh + i%4; only heads < GQ (i < 4) are real
  if (hh == 0 && ln < GQ) { wm[wave][ln] = m; wl[wave][ln] = l; }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int h = 4 * hh + i;
    if (h < GQ)
#pragma unroll
      for (int t = 0; t < NT; ++t) wo[wave][h][32 * t + ln] = o[t][i];
  }
  __syncthreads();
  // the four waves merged (exact rule with a common reference); this
  // workgroup's partial per head: [M, L, O / L]
  const int Hq = a.Hkv * a.G;
  for (int i = tid; i < GQ * D; i += 256) {
    const int h = i / D, d = i - h * D;
    const float M = fmaxf(fmaxf(wm[0][h], wm[1][h]), fmaxf(wm[2][h], wm[3][h]));
    float L = 0.f, O = 0.f;
    if (M != kNegInf) {
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float f = wm[w][h] == kNegInf ? 0.f : exp2f(wm[w][h] - M);
        L += wl[w][h] * f;
        O += wo[w][h][d] * f;
      }
    }
    float* pp = a.part + ((((int64_t)layer * a.B + b) * Hq + h0 + h) * a.nsplit + split) * (D + 2);
    pp[2 + d] = L > 0.f ? O / L : 0.f;
    if (d == 0) { pp[0] = M; pp[1] = L; }
  }
}

// Merge of the selected-block partials (exact rule with a common reference)
// and the gate: g = sigmoid(<q_h, w_h>); an empty sparse set leaves the window
// branch.  One wave per (layer, sequence, query head), lane = head dims.
template <int D>
__global__ __launch_bounds__(256) void hs_decode_gate_kernel(const HsDecArgs a) {
  constexpr int DP = D / 64;
  const int Hq = a.Hkv * a.G;
  const int w = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (w >= a.nlayer * a.B * Hq) return;
  const int h = w % Hq, b = (w / Hq) % a.B, layer = w / (Hq * a.B);
  const int ns = a.nsplit;
  const float* pp = a.part + (((int64_t)layer * a.B + b) * Hq + h) * ns * (D + 2);
  float M = kNegInf;
  for (int s = 0; s < ns - 1; ++s) M = fmaxf(M, pp[s * (D + 2)]);
  float L = 0.f, O[DP];
#pragma unroll
  for (int e = 0; e < DP; ++e) O[e] = 0.f;
  if (M != kNegInf)
    for (int s = 0; s < ns - 1; ++s) {
      const float ms = pp[s * (D + 2)];
      const float f = ms == kNegInf ? 0.f : exp2f(ms - M) * pp[s * (D + 2) + 1];
      L += f;
#pragma unroll
      for (int e = 0; e < DP; ++e) O[e] += f * pp[s * (D + 2) + 2 + DP * lane + e];
    }
  const float* pw = pp + (ns - 1) * (D + 2) + 2;
  const uint16_t* qr = a.q[layer] + (int64_t)b * a.q_sb + (int64_t)h * a.q_sh;
  const float* gw = a.gate_w[layer] + (int64_t)h * D;
  float z = 0.f;
#pragma unroll
  for (int e = 0; e < DP; ++e) z += bf16_to_f32(qr[DP * lane + e]) * gw[DP * lane + e];
  z = wave_sum(z);
  const float gt = 1.f / (1.f + __expf(-z));
  const bool empty = !(L > 0.f);
  const int64_t orow = (int64_t)b * a.o_sb + (int64_t)h * a.o_sh;
#pragma unroll
  for (int e = 0; e < DP; ++e) {
    const int d = DP * lane + e;
    const float ow = pw[d];
    const float out = empty ? ow : gt * (O[e] / L) + (1.f - gt) * ow;
    if (a.o_f32) ((float*)a.o[layer])[orow + d] = out;
    else ((uint16_t*)a.o[layer])[orow + d] = f32_to_bf16(out);
  }
}

int hs_decode_splits(int topk) { return (topk + 3) / 4 + 1; }

hipError_t launch_hs_decode_sparse(int D, const HsDecArgs& a, hipStream_t s) {
  // at most 8 query heads per workgroup
  const int gq = a.G <= 8 ? a.G : 8;
  if (a.G % gq != 0) return hipErrorInvalidValue;
  if (a.nsplit != hs_decode_splits(a.topk)) return hipErrorInvalidValue;
  const int64_t grid = (int64_t)a.nlayer * a.B * a.Hkv * (a.G / gq) * a.nsplit;
  if (grid == 0) return hipSuccess;
  hipError_t e = hipErrorInvalidValue;   // group size not a power of two up to 16
#define HYS_HS_LAUNCH(DD, GG) \
  if (D == DD && gq == GG) { hipLaunchKernelGGL((hs_decode_sparse_kernel<DD, GG>), dim3((unsigned)grid), dim3(256), 0, s, a); e = hipGetLastError(); }
  HYS_HS_LAUNCH(128, 1) HYS_HS_LAUNCH(128, 2) HYS_HS_LAUNCH(128, 4) HYS_HS_LAUNCH(128, 8)
  HYS_HS_LAUNCH(64, 1) HYS_HS_LAUNCH(64, 2) HYS_HS_LAUNCH(64, 4) HYS_HS_LAUNCH(64, 8)
#undef HYS_HS_LAUNCH
  if (e != hipSuccess) return e;
  const int64_t waves = (int64_t)a.nlayer * a.B * a.Hkv * a.G;
  if (D == 128)
    hipLaunchKernelGGL((hs_decode_gate_kernel<128>), dim3((unsigned)((waves + 3) / 4)), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((hs_decode_gate_kernel<64>), dim3((unsigned)((waves + 3) / 4)), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace hys
