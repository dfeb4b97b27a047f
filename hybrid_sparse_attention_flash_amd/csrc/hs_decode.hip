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
// native 16-byte vector (register arrays of HIP's uint4 wrapper struct end up in scratch)
typedef unsigned int hs_u32x4 __attribute__((ext_vector_type(4)));

// eight bf16 of a key row as fp32
__device__ __forceinline__ void bf16x8_to_f32(hs_u32x4 r, float (&x)[8]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = __builtin_bit_cast(float, r[i] << 16);
    x[2 * i + 1] = __builtin_bit_cast(float, r[i] & 0xffff0000u);
  }
}
}  // namespace

// GQ: query heads per workgroup, a compile-time constant so the per-head
// softmax state stays in registers; a KV head's a.G query heads are split
// into a.G / GQ sub-groups, one workgroup each
template <int D, int GQ>
__global__ __launch_bounds__(256) void hs_decode_sparse_kernel(const HsDecArgs a) {
  constexpr int DP = D / 64;                 // head dims per lane in the P V phase
  __shared__ __attribute__((aligned(16))) uint32_t qs[kHsGmax][D / 2];   // bf16 pairs
  __shared__ __attribute__((aligned(16))) float ps[4][kHsGmax][64];
  __shared__ float wm[4][kHsGmax], wl[4][kHsGmax];
  __shared__ __attribute__((aligned(16))) float wo[4][kHsGmax][D];
  __shared__ int sel[kHsKmax];

  // wave index as a wave-uniform value, so chunk and row addresses stay scalar
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
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
  // ---- the group's queries (fp32) and the selected blocks
  const uint16_t* qb = a.q[layer] + (int64_t)b * a.q_sb;
  for (int i = tid; i < kHsGmax * (D / 2); i += 256) {
    const int h = i / (D / 2), d2 = i - h * (D / 2);
    qs[h][d2] = h < GQ ? *(const uint32_t*)(qb + (int64_t)(h0 + h) * a.q_sh + 2 * d2) : 0u;
  }
  if (tid < kHsKmax) sel[tid] = tid < a.topk ? a.idx[(int64_t)b * a.idx_sb + tid] : -1;
  __syncthreads();

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
  {
    const int br = win ? 1 : 0;
    const int c0 = win ? 0 : 4 * split;
    const int nchunk = win ? (n - wstart + 63) / 64 : min(a.topk, c0 + 4);
    float m[GQ], l[GQ], o[GQ][DP];
#pragma unroll
    for (int h = 0; h < GQ; ++h) {
      m[h] = kNegInf;
      l[h] = 0.f;
#pragma unroll
      for (int e = 0; e < DP; ++e) o[h][e] = 0.f;
    }
    for (int c = c0 + wave; c < nchunk; c += 4) {
      // keeps the query reads from LDS inside the loop (hoisted, G x D of them
      // would not fit in registers)
      __asm__ volatile("" ::: "memory");
      // key rows of chunk c: position x = 0..63 (uniform per chunk for the P V phase)
      const int blk = br == 0 ? __builtin_amdgcn_readfirstlane(sel[c]) : 0;   // uniform: scalar row addresses
      auto krow = [&](int x, bool& valid) -> const uint16_t* {
        if (br == 0) {
          const int j = blk * 64 + x;
          valid = blk >= 0 && j < n;
          return kc + (int64_t)(valid ? j : 0) * a.k_st;
        }
        const int t = wstart + c * 64 + x;
        valid = t < n;
        if (t == n - 1) return kn;
        return kr + (int64_t)((valid ? t : 0) % W) * a.r_st;
      };
      auto vrow = [&](int x, bool& valid) -> const uint16_t* {
        if (br == 0) {
          const int j = blk * 64 + x;
          valid = blk >= 0 && j < n;
          return vc + (int64_t)(valid ? j : 0) * a.v_st;
        }
        const int t = wstart + c * 64 + x;
        valid = t < n;
        if (t == n - 1) return vn;
        return vr + (int64_t)((valid ? t : 0) % W) * a.r_st;
      };
      // logits, lane = key: the key row's loads are all issued before use
      bool kvalid;
      const uint16_t* kp = krow(lane, kvalid);
      hs_u32x4 kraw[D / 8];
#pragma unroll
      for (int p = 0; p < D / 8; ++p) kraw[p] = *(const hs_u32x4*)(kp + 8 * p);
      float s[GQ];
#pragma unroll
      for (int h = 0; h < GQ; ++h) {
        float acc = 0.f;
#pragma unroll
        for (int p = 0; p < D / 8; ++p) {
          const hs_u32x4 q4 = *(const hs_u32x4*)&qs[h][4 * p];
          // bf16 pairs widened in place (a bf16 is the upper half of its fp32);
          // v_dot2c_f32_bf16 gave wrong sums here although it is exact alone
#pragma unroll
          for (int i = 0; i < 4; ++i)
            acc += __builtin_bit_cast(float, kraw[p][i] << 16) * __builtin_bit_cast(float, q4[i] << 16) +
                   __builtin_bit_cast(float, kraw[p][i] & 0xffff0000u) * __builtin_bit_cast(float, q4[i] & 0xffff0000u);
        }
        s[h] = acc;
      }
      // online softmax per head over the chunk (base 2)
#pragma unroll
      for (int h = 0; h < GQ; ++h) {
        const float sv = kvalid ? s[h] * c2 : kNegInf;
        const float mn = fmaxf(m[h], wave_max(sv));
        const float alpha = mn == kNegInf ? 1.f : exp2f(m[h] - mn);
        const float pv = sv == kNegInf ? 0.f : exp2f(sv - mn);
        l[h] = l[h] * alpha + wave_sum(pv);
        m[h] = mn;
#pragma unroll
        for (int e = 0; e < DP; ++e) o[h][e] *= alpha;
        ps[wave][h][lane] = pv;
      }
      // P V, lane = head dims [DP lane, +DP), keys in batches of VB whose row
      // loads are issued together; invalid keys read a clamped row with p = 0.
      // ps is read by the wave that wrote it.
      constexpr int VB = 32;                   // keys per batch of V-row loads
#pragma unroll
      for (int x0 = 0; x0 < 64; x0 += VB) {
        uint32_t vraw[VB];
#pragma unroll
        for (int i = 0; i < VB; ++i) {
          bool vvalid;
          const uint16_t* vp = vrow(x0 + i, vvalid);
          vraw[i] = DP == 2 ? *(const uint32_t*)(vp + 2 * lane) : (uint32_t)vp[lane];
        }
#pragma unroll
        for (int h = 0; h < GQ; ++h) {
#pragma unroll
          for (int i4 = 0; i4 < VB / 4; ++i4) {
            const f32x4 p4 = *(const f32x4*)&ps[wave][h][x0 + 4 * i4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const uint32_t vv = vraw[4 * i4 + j];
              o[h][0] += p4[j] * __builtin_bit_cast(float, vv << 16);
              if (DP == 2) o[h][DP - 1] += p4[j] * __builtin_bit_cast(float, vv & 0xffff0000u);
            }
          }
        }
      }
    }
    // merge the four waves' partials (exact rule with a common reference)
#pragma unroll
    for (int h = 0; h < GQ; ++h) {
      if (lane == 0) { wm[wave][h] = m[h]; wl[wave][h] = l[h]; }
#pragma unroll
      for (int e = 0; e < DP; ++e) wo[wave][h][DP * lane + e] = o[h][e];
    }
    __syncthreads();
    // this workgroup's partial per head: [M, L, O / L]
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
