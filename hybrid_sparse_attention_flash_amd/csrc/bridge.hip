// KV Bridging projection for HySparse2 (gfx950): the cross-decoder full
// layer's K and V projected from the self-decoder full layer's hidden states
// (airebao HySparse2 news, outer KV Bridging paragraph; demingchina
// commentary, section 02) and written straight into the shared fp8 e4m3 MQA
// cache (airebao key-data table), so that KV is materialised once.
//
//   K[b,t,:] = h[b,t,:] W_k^T,  V[b,t,:] = h[b,t,:] W_v^T      (W: [Hkv*D, d_model])
//   code = e4m3(clamp(x * (1/s), -448, 448)), round to nearest even
//
// One GEMM per tile with both operands contiguous along d_model: C^T = W h^T
// on v_mfma_f32_32x32x16_bf16 (A = 32 rows of W, B = 32 tokens of h).  The
// projection reads each hidden state once and is bound by that HBM stream, so
// the kernel is laid out to keep it flowing:
//   * a workgroup of 4 waves (one per SIMD) owns 256 tokens x 256 outputs
//     (128 of K and the same 128 of V); each wave holds all 256 outputs of
//     its own 64 tokens, 16 accumulator blocks in the accumulation registers;
//   * h goes from HBM straight into registers in MFMA operand layout, three
//     64-column chunks ahead of the multiply (96 KB per CU in flight): lane
//     (l%32, l/32) of a wave loads 32 consecutive columns [32 (l/32), +32) of
//     token l%32 per chunk, and MFMA step j of the chunk contracts columns
//     32 (l/32) + 8 j + [0, 8) (the contraction order inside a chunk is free
//     as long as W is read in the same order);
//   * W (the same 2 * 128 rows for every token tile, L2-resident) is staged
//     per chunk through a two-stage LDS ring shared by the four waves.
// The epilogue scales, clamps and converts in registers and stores four
// consecutive dims of one token as one dword; max |x| is reduced per wave and
// raised with an atomic max.
#include "common.h"
#include "kernels.h"

namespace hys {

namespace {
constexpr int kBrTok = 256;                 // tokens per workgroup (64 per wave)
constexpr int kBrOut = 256;                 // outputs per workgroup (128 K + 128 V)
constexpr int kBrK = 64;                    // d_model columns per chunk
constexpr int kBrRow = kBrK + 8;            // LDS row stride (bf16 elements): conflict-free b128 reads
constexpr int kBrStage = kBrOut * kBrRow;   // elements per W stage
constexpr int kBrStages = 3;                // W ring depth
constexpr int kBrSlots = 3;                 // h chunks held per lane: the current one + 2 in flight
// native 16-byte vector (HIP's uint4 wrapper struct keeps register arrays of it in scratch here)
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ bf16x8 frag(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// instruction classes of __builtin_amdgcn_sched_group_barrier
constexpr int kSgMfma = 0x008, kSgVmemRead = 0x020, kSgDsRead = 0x100, kSgDsWrite = 0x200;
}  // namespace

__global__ __launch_bounds__(256, 1) void kv_bridge_kernel(const BridgeArgs a) {
  // W ring, then one all-zero stage
  __shared__ __attribute__((aligned(16))) uint16_t lds[(kBrStages + 1) * kBrStage];
  uint16_t* const zst = lds + kBrStages * kBrStage;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, hh = lane >> 5, ln = lane & 31;
  const int64_t rows = (int64_t)a.B * a.L;
  const int ntt = (int)((rows + kBrTok - 1) / kBrTok);
  const int ny = a.Hkv * a.D / 128;
  // the ny output tiles of one token tile go to one XCD (workgroup ids are
  // dealt round-robin over the 8 XCDs), so their h reads meet in one L2
  const int bid = blockIdx.x, xcd = bid & 7, slot = bid >> 3;
  const int tile = (slot / ny) * 8 + xcd, nt = slot % ny;
  if (tile >= ntt) return;
  const int64_t tok0 = (int64_t)tile * kBrTok;
  const int nchunk = a.d_model / kBrK;

  // ---- h rows of this lane (rows past the end are clamped: loaded, never stored)
  const uint16_t* hp[2];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
    int64_t g = tok0 + 64 * wave + 32 * mb + ln;
    if (g >= rows) g = rows - 1;
    const int64_t b = g / a.L, t = g - b * a.L;
    hp[mb] = (const uint16_t*)a.h + b * a.h_sb + t * a.h_st + 32 * hh;
  }
  // ---- W staging: 2048 16-byte units per chunk, 8 per thread; unit u of
  // thread t is row 32 u + t/8 of the 256 (K rows, then V rows), columns 8 (t%8) + [0, 8)
  // (uniform base + 32-bit lane offset: the loads take the scalar-base form)
  const char* wbk = (const char*)a.w_k + (int64_t)nt * 128 * a.d_model * 2;
  const char* wbv = (const char*)a.w_v + (int64_t)nt * 128 * a.d_model * 2;
  uint32_t woff[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) woff[u] = (uint32_t)(((tid >> 3) + 32 * u) * a.d_model * 2 + (tid & 7) * 16);
  const int lbase = (tid >> 3) * kBrRow + (tid & 7) * 8;
  // W fragment of block nb, step j: row 32 nb + ln, columns 32 hh + 8 j + [0, 8)
  const int rbase = ln * kBrRow + 32 * hh;

  u32x4 hbuf[kBrSlots][2][4];
  u32x4 wreg[8];
  u32x4 wf[2][8];
  f32x16 acc[8][2];
#pragma unroll
  for (int nb = 0; nb < 8; ++nb)
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[nb][mb][i] = 0.f;

  if (nchunk % kBrSlots != 0) {
    for (int i = tid * 8; i < kBrStage; i += 256 * 8) *(u32x4*)&zst[i] = u32x4{0u, 0u, 0u, 0u};
  }
  // ---- prologue: W chunk 0 into stage 0, W chunk 1 into registers, h
  // chunks 0 and 1 in flight, step 0 fragments of chunk 0.  d_model >= 64,
  // so nchunk >= 1; prefetches past the last chunk re-read the last chunk
  // (in bounds) and are never used.
#pragma unroll
  for (int u = 0; u < 8; ++u) wreg[u] = *(const u32x4*)((u < 4 ? wbk : wbv) + woff[u & 3]);
#pragma unroll
  for (int u = 0; u < 8; ++u) *(u32x4*)&lds[lbase + u * 32 * kBrRow] = wreg[u];
  {
    const int64_t c1 = min(1, nchunk - 1) * kBrK * 2;
#pragma unroll
    for (int u = 0; u < 8; ++u) wreg[u] = *(const u32x4*)((u < 4 ? wbk : wbv) + c1 + woff[u & 3]);
  }
#pragma unroll
  for (int s = 0; s < kBrSlots - 1; ++s) {
    const int cs = min(s, nchunk - 1) * kBrK;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int p = 0; p < 4; ++p) hbuf[s][mb][p] = *(const u32x4*)(hp[mb] + cs + 8 * p);
  }
  __syncthreads();
#pragma unroll
  for (int nb = 0; nb < 8; ++nb) wf[0][nb] = *(const u32x4*)&lds[rbase + 32 * nb * kBrRow];

  // ---- main loop over whole groups of kBrSlots chunks.  Chunk c: write W(c+1) (registers) into stage (c+1)%3,
  // load W(c+2) and h(c+2), multiply four 16-column steps, each reading the
  // next step's W fragments; after step 1 a barrier publishes stage (c+1)%3,
  // which step 3 reads for chunk c+1.  Stage (c+1)%3 was last read in chunk
  // c-2 (and chunk c-3's step 3), finished by every wave before chunk c-1's
  // barrier.
  for (int c0 = 0; c0 < nchunk; c0 += kBrSlots) {
#pragma unroll
    for (int s = 0; s < kBrSlots; ++s) {
      const int c = c0 + s;
      const int st_cur = c % kBrStages, st_nxt = (c + 1) % kBrStages;
      uint16_t* Wn = lds + st_nxt * kBrStage;
#pragma unroll
      for (int u = 0; u < 8; ++u) *(u32x4*)&Wn[lbase + u * 32 * kBrRow] = wreg[u];
      {
        const int c2 = min(c + 2, nchunk - 1) * kBrK;
        const char* bk = wbk + (int64_t)c2 * 2;
        const char* bv = wbv + (int64_t)c2 * 2;
#pragma unroll
        for (int u = 0; u < 8; ++u) wreg[u] = *(const u32x4*)((u < 4 ? bk : bv) + woff[u & 3]);
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int p = 0; p < 4; ++p)
            hbuf[(s + kBrSlots - 1) % kBrSlots][mb][p] = *(const u32x4*)(hp[mb] + c2 + 8 * p);
      }
      // chunks past the end (the loop runs whole groups of kBrSlots) read
      // their fragments from the zero stage, so their products add exactly 0
      const uint16_t* Wc = c < nchunk ? lds + st_cur * kBrStage : zst;
      const uint16_t* Wr = c + 1 < nchunk ? Wn : zst;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (j == 2) __syncthreads();
        // fragments of the next step: same stage, or step 0 of chunk c + 1
        const uint16_t* src = j < 3 ? Wc + 8 * (j + 1) : Wr;
#pragma unroll
        for (int nb = 0; nb < 8; ++nb) {
          acc[nb][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(frag(wf[j & 1][nb]), frag(hbuf[s][0][j]),
                                                              acc[nb][0], 0, 0, 0);
          acc[nb][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(frag(wf[j & 1][nb]), frag(hbuf[s][1][j]),
                                                              acc[nb][1], 0, 0, 0);
          wf[(j + 1) & 1][nb] = *(const u32x4*)&src[rbase + 32 * nb * kBrRow];
        }
        if (j == 0) {
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            __builtin_amdgcn_sched_group_barrier(kSgDsWrite, 1, 0);
            __builtin_amdgcn_sched_group_barrier(kSgMfma, 1, 0);
          }
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            __builtin_amdgcn_sched_group_barrier(kSgVmemRead, 2, 0);
            __builtin_amdgcn_sched_group_barrier(kSgMfma, 1, 0);
            __builtin_amdgcn_sched_group_barrier(kSgDsRead, 1, 0);
          }
        } else {
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            __builtin_amdgcn_sched_group_barrier(kSgMfma, 2, 0);
            __builtin_amdgcn_sched_group_barrier(kSgDsRead, 1, 0);
          }
        }
      }
    }
  }

  // ---- epilogue: lane (ln, hh) of block (nb, mb) holds outputs
  // 32 nb + 8 (v/4) + 4 hh + v%4 (v = 0..15) of token tok0 + 64 wave + 32 mb + ln
  float amk = 0.f, amv = 0.f;
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
    const int64_t g = tok0 + 64 * wave + 32 * mb + ln;
    const bool valid = g < rows;
    const int64_t b = valid ? g / a.L : 0, t = valid ? g - b * a.L : 0;
    const int64_t tok_off = b * a.o_sb + t * a.o_st;
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) {
      const bool isv = nb >= 4;
      const float inv = isv ? a.inv_v : a.inv_k;
      uint8_t* outp = (uint8_t*)(isv ? a.v_out : a.k_out) + tok_off;
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        float y[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float x = acc[nb][mb][4 * q4 + e];
          if (valid) {
            if (isv) amv = fmaxf(amv, fabsf(x));
            else amk = fmaxf(amk, fabsf(x));
          }
          y[e] = fminf(fmaxf(x * inv, -448.f), 448.f);
        }
        uint32_t w = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);
        w = __builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], w, true);
        const int o = nt * 128 + 32 * (nb & 3) + 8 * q4 + 4 * hh;   // output dim in [0, Hkv*D)
        const int head = o / a.D, d = o - head * a.D;
        if (valid) *(uint32_t*)(outp + (int64_t)head * a.o_sh + d) = w;
      }
    }
  }
  if (a.amax) {
    amk = wave_max(amk);
    amv = wave_max(amv);
    // non-negative floats order like their bit patterns
    if (lane == 0) {
      atomicMax((unsigned int*)&a.amax[0], __float_as_uint(amk));
      atomicMax((unsigned int*)&a.amax[1], __float_as_uint(amv));
    }
  }
}

hipError_t launch_kv_bridge(const BridgeArgs& a, hipStream_t s) {
  const int64_t rows = (int64_t)a.B * a.L;
  if (rows == 0) return hipSuccess;
  const int64_t ntt = (rows + kBrTok - 1) / kBrTok;
  const int64_t ny = a.Hkv * a.D / 128;
  const int64_t grid = ((ntt + 7) / 8) * 8 * ny;
  if (grid > INT32_MAX) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(kv_bridge_kernel, dim3((unsigned)grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace hys
