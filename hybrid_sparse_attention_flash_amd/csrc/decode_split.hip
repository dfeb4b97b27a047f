// HySparse2 decode, full layer, fp8 e4m3 cache with D = 128: the split-K
// kernel in its all-compute form.
//
// Decoding keeps the whole cache, so the full layer of a decode step is one
// pass over it and memory bandwidth bounds it (QbitAI HySparse article,
// background section; airebao HySparse2 news, key-data table: decode at 1M
// tokens with an FP8 KV cache).  Each workgroup takes a contiguous share of
// the 64-key tiles of one sequence, as the staged kernel in decode.hip does,
// but without a staging role:
//
//  * fp8 tiles go HBM -> LDS with global_load_lds_dwordx4 (each lane moves 16
//    bytes, a wave 1 KiB, all four waves a quarter of each tile), into a ring
//    of four stages.  A stage is busy only while its tile's fragments are
//    read into registers (the first thing a tile's compute does): a barrier
//    after the reads hands it to the loads of the tile four ahead, so four
//    tiles are in flight while one is computed.  No registers hold data in
//    flight and nothing is converted on the way in.
//  * Every wave computes: wave w takes keys [32(w/2), +32) of each tile for
//    query heads [32(w%2), +32) (the MFMA N dimension).  K fragments are read
//    with ds_read_b128 and decoded to bf16 in registers (one
//    v_cvt_scalef32_pk_bf16_fp8 per two values); V^T fragments come straight
//    from the fp8 rows by ds_read_b64_tr_b8 (within each 16-lane slice, lane
//    j receives byte j%8 of the 8-byte chunk that slice lane 2e + j/8
//    addresses, as element e), then are decoded the same way.
//  * S^T = K q^T and O^T += V^T P^T on v_mfma_f32_32x32x16_bf16 with the
//    lazily moved softmax reference of the other attention kernels; the
//    per-key maximum over heads (the token score) is reduced in registers
//    (colmax16_swap / colmax16_dpp) and over the two head halves in LDS.
//  * Issue order is laid out by hand: an MFMA that has to wait for the busy
//    matrix pipe holds up the SIMD's VALU issue (measured: one wave of
//    back-to-back MFMAs and one of VALU on a SIMD take longer than the two
//    run one after the other), so every MFMA is followed by independent
//    VALU work of this wave - fragment decodes under the S^T chain, the
//    softmax's second half, the token score and the row sum under O^T.
//  * The two waves of a head half merge their (m, l, O) through LDS at the
//    end (exact LSE rule), so each workgroup leaves one partial per head, in
//    the layout decode_merge_kernel reads.
#include "common.h"
#include "kernels.h"
#include "decode_split.h"
#include <type_traits>

namespace hys {
namespace {

typedef int ds_v2i32 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) ds_v2i32 ds_lds_v2i32;
typedef __attribute__((address_space(3))) void ds_lds_void;

constexpr int kDsD = 128;             // head dim
constexpr int kDsRow = kDsD;          // bytes per fp8 key row in LDS
constexpr int kDsTile = 64 * kDsRow;  // bytes per operand and stage

// chunk x (16 bytes) of key row r is stored at chunk x ^ swz(r).  K: the 16
// rows one ds_read_b128 cycle addresses fall in distinct banks (64 banks;
// and the 8 of a 32-bank cycle).  V: likewise for the transposing reads'
// rows, 32 lanes per cycle (64 banks) or 16 (32 banks).  Both depend on the
// row mod 16 only.
__device__ __forceinline__ int ds_swz_k(int r) { return (r ^ (r >> 3)) & 7; }
__device__ __forceinline__ int ds_swz_v(int r) { return (r ^ (4 * (r >> 3))) & 7; }

// this wave's LDS accesses are done and at most PENDING of its vector memory
// operations are still in flight (the LDS loads complete in issue order, so
// these are the newest); then the workgroup barrier
template <int PENDING>
__device__ __forceinline__ void ds_tile_barrier() {
  static_assert(PENDING >= 0 && PENDING < 16, "vmcnt field");
  __builtin_amdgcn_s_waitcnt(0x0070 | PENDING);   // vmcnt(PENDING) lgkmcnt(0)
  asm volatile("s_barrier" ::: "memory");
}

// Row maxima of one 32 x 32 MFMA result block over its columns: v[i] is
// element i of the block in the C layout (lane l holds rows 8(i/4) +
// 4(l/32) + i%4 of column l%32), and the result is the maximum over the 32
// columns for two rows, r0 and r0 + 1, with r0 = 16(R%2) + 8(j/8) + 4(R/2) +
// 2((j/4)%2) for R = l/16, j = l%16 (all four lanes of a quad hold the same
// pair).  The same reduce-scatter as colmax32 on half the registers, in two
// parts that callers may place apart: colmax16_swap(v[x], v[x + 8]) for
// x = 0..7 (v_permlane16_swap over lanes 16 apart) gives w[x], then
// colmax16_dpp(w) (bank-masked DPP row_mirror and row_half_mirror steps and
// a quad all-reduce).
__device__ __forceinline__ float colmax16_swap(float a, float b) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  return fmax_nc(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ f32x2 colmax16_dpp(float (&w)[8]) {
  // every DPP read is at least two wait states after the write of its source
  asm("s_nop 1\n\t"
      "v_max_f32_dpp %0, %0, %0 row_mirror row_mask:0xf bank_mask:0x3\n\t"
      "v_max_f32_dpp %0, %4, %4 row_mirror row_mask:0xf bank_mask:0xc\n\t"
      "v_max_f32_dpp %1, %1, %1 row_mirror row_mask:0xf bank_mask:0x3\n\t"
      "v_max_f32_dpp %1, %5, %5 row_mirror row_mask:0xf bank_mask:0xc\n\t"
      "v_max_f32_dpp %2, %2, %2 row_mirror row_mask:0xf bank_mask:0x3\n\t"
      "v_max_f32_dpp %2, %6, %6 row_mirror row_mask:0xf bank_mask:0xc\n\t"
      "v_max_f32_dpp %3, %3, %3 row_mirror row_mask:0xf bank_mask:0x3\n\t"
      "v_max_f32_dpp %3, %7, %7 row_mirror row_mask:0xf bank_mask:0xc\n\t"
      "v_max_f32_dpp %0, %0, %0 row_half_mirror row_mask:0xf bank_mask:0x5\n\t"
      "v_max_f32_dpp %0, %2, %2 row_half_mirror row_mask:0xf bank_mask:0xa\n\t"
      "v_max_f32_dpp %1, %1, %1 row_half_mirror row_mask:0xf bank_mask:0x5\n\t"
      "v_max_f32_dpp %1, %3, %3 row_half_mirror row_mask:0xf bank_mask:0xa\n\t"
      "s_nop 1\n\t"
      "v_max_f32_dpp %0, %0, %0 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf\n\t"
      "v_max_f32_dpp %1, %1, %1 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf\n\t"
      "s_nop 1\n\t"
      "v_max_f32_dpp %0, %0, %0 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
      "v_max_f32_dpp %1, %1, %1 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf"
      : "+v"(w[0]), "+v"(w[1]), "+v"(w[2]), "+v"(w[3])
      : "v"(w[4]), "v"(w[5]), "v"(w[6]), "v"(w[7]));
  const f32x2 o = {w[0], w[1]};
  return o;
}

// One 16-byte-per-lane LDS-direct load (global_load_lds_dwordx4): lane l's
// 16 bytes from base + voff (saddr form) or from addr land at LDS byte lds +
// 16 l.  Written as asm so the compiler does not track these LDS writes:
// every wait on them is the explicit vmcnt of ds_tile_barrier (the loads
// complete in issue order), and the memory clobber keeps LDS accesses from
// moving across them.  No register receives a result.
__device__ __forceinline__ void dma16(const void* base, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :: "v"(voff), "s"(base), "s"(lds) : "memory", "m0");
}
__device__ __forceinline__ void dma16(const void* addr, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :: "v"(addr), "s"(lds) : "memory", "m0");
}

// this wave's LDS reads have returned; then the workgroup barrier
__device__ __forceinline__ void ds_reads_barrier() {
  __builtin_amdgcn_s_waitcnt(0xc07f);             // lgkmcnt(0)
  asm volatile("s_barrier" ::: "memory");
}

// two e4m3 bytes pairs of a dword -> the four bf16 pairs of an MFMA fragment
__device__ __forceinline__ uint4 fp8x8_to_bf16x8(uint32_t lo, uint32_t hi) {
  uint4 r;
  r.x = fp8x2_to_bf16x2(lo, false);
  r.y = fp8x2_to_bf16x2(lo, true);
  r.z = fp8x2_to_bf16x2(hi, false);
  r.w = fp8x2_to_bf16x2(hi, true);
  return r;
}

// two workgroups share a CU (65 KB of LDS each)
__global__ __launch_bounds__(256, 2) void decode_split_fp8_kernel(const DecArgs a) {
  // one array per operand and stage, every access naming one statically (the
  // tile loop is unrolled by four): the compiler then tells the loads into
  // one stage from the reads of another and keeps them in flight
  __shared__ __attribute__((aligned(1024))) unsigned char K0[kDsTile];
  __shared__ __attribute__((aligned(1024))) unsigned char K1[kDsTile];
  __shared__ __attribute__((aligned(1024))) unsigned char K2[kDsTile];
  __shared__ __attribute__((aligned(1024))) unsigned char K3[kDsTile];
  __shared__ __attribute__((aligned(1024))) unsigned char V0[kDsTile];
  __shared__ __attribute__((aligned(1024))) unsigned char V1[kDsTile];
  __shared__ __attribute__((aligned(1024))) unsigned char V2[kDsTile];
  __shared__ __attribute__((aligned(1024))) unsigned char V3[kDsTile];
  __shared__ __attribute__((aligned(16))) float red[2][2][64];   // [tile parity][head half][key]

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hh = lane >> 5, ln = lane & 31;
  const int kh = wave >> 1, hb = wave & 1;   // key half of each tile, head half
  const int bid = blockIdx.x;
  const int s = bid % a.nsplit;
  const int rest = bid / a.nsplit;
  const int b = rest % a.B;
  const int layer = rest / a.B;
  const int n = a.lens[b];
  const int ntiles = (n + 63) / 64;
  const int per = (ntiles + a.nsplit - 1) / a.nsplit;
  const int t0 = s * per, t1 = min(ntiles, t0 + per);
  // the ints a later launch of the step needs cleared (the top-k's histograms)
  if (bid == 0 && a.zero)
    for (int64_t i = tid; i < a.zero_n; i += 256) a.zero[i] = 0;

  // ---- tile loads: instruction u of wave w fills rows 16w + 8u + (0..7), lane
  // L the row's chunk slot L%8 with source chunk (L%8) ^ swz(row) ----------
  const uint32_t kst = (uint32_t)a.k_st, vst = (uint32_t)a.v_st;   // bytes per key row
  const unsigned char* kg = (const unsigned char*)a.k + (int64_t)b * a.k_sb;
  const unsigned char* vg = (const unsigned char*)a.v + (int64_t)b * a.v_sb;
  const int drow = 16 * wave + (lane >> 3);
  const uint32_t ck0 = (uint32_t)(((lane & 7) ^ ds_swz_k(drow)) * 16), ck1 = (uint32_t)(((lane & 7) ^ ds_swz_k(drow + 8)) * 16);
  const uint32_t cv0 = (uint32_t)(((lane & 7) ^ ds_swz_v(drow)) * 16), cv1 = (uint32_t)(((lane & 7) ^ ds_swz_v(drow + 8)) * 16);
  const uint32_t lk0 = (uint32_t)drow * kst + ck0, lk1 = (uint32_t)(drow + 8) * kst + ck1;
  const uint32_t lv0 = (uint32_t)drow * vst + cv0, lv1 = (uint32_t)(drow + 8) * vst + cv1;
  // (64 key rows span less than 2^32 bytes: checked at launch)
  auto load_tile = [&](int t, unsigned char* Kd, unsigned char* Vd) __attribute__((always_inline)) {
    const unsigned char* kt = kg + (int64_t)t * 64 * a.k_st;
    const unsigned char* vt = vg + (int64_t)t * 64 * a.v_st;
    // LDS byte addresses of this wave's two 1 KiB blocks of each operand
    const uint32_t kd0 = (uint32_t)(uintptr_t)(ds_lds_void*)(Kd + (2 * wave) * 1024);
    const uint32_t vd0 = (uint32_t)(uintptr_t)(ds_lds_void*)(Vd + (2 * wave) * 1024);
    if (t * 64 + 63 < n) {
      dma16(kt, lk0, kd0);
      dma16(kt, lk1, kd0 + 1024);
      dma16(vt, lv0, vd0);
      dma16(vt, lv1, vd0 + 1024);
    } else {
      // the last tile: rows past the last key repeat the last key (their
      // logits are masked, so their probabilities are exactly 0)
      const uint32_t rmax = (uint32_t)(n - 1 - t * 64);
      const uint32_t r0 = min((uint32_t)drow, rmax), r1 = min((uint32_t)drow + 8u, rmax);
      dma16(kt + (r0 * kst + ck0), kd0);
      dma16(kt + (r1 * kst + ck1), kd0 + 1024);
      dma16(vt + (r0 * vst + cv0), vd0);
      dma16(vt + (r1 * vst + cv1), vd0 + 1024);
    }
  };

  // ---- query fragments (B of S^T).  The K read of pair p gives a lane 16
  // bytes of its key at d = 16(2p + hh) ..; k-step 2p + e takes bytes 8e ..
  // 8e + 7 of them, so q is read in the same order: q[head][32p + 16hh + 8e ..]
  const int head = 32 * hb + ln;
  const bool hvalid = head < a.Hq;
  const uint16_t* qb = (const uint16_t*)a.q[layer] + (int64_t)b * a.q_sb + (int64_t)(hvalid ? head : 0) * a.q_sh;
  // (a padding head reads head 0's row: its logits are masked to -inf and its
  // partial is not written).  The fragments land before any tile load is
  // issued, so no wait for them waits for tiles as well.
  bf16x8 qf[8];
#pragma unroll
  for (int st = 0; st < 8; ++st) qf[st] = as_bf16x8(*(const uint4*)(qb + 32 * (st >> 1) + 16 * hh + 8 * (st & 1)));
  __builtin_amdgcn_s_waitcnt(0x3f70);             // vmcnt(0)
#pragma unroll
  for (int st = 0; st < 8; ++st) asm volatile("" : "+v"(qf[st]));

  // per-lane LDS byte offsets inside a stage.  K, pair p: row 32kh + ln,
  // chunk 2p + hh, so the base XOR 32p.  V^T, d block db, k-step kc: slice
  // lane i = lane%16 addresses row 32kh + 16kc + 4hh + (e%4) + 8(e/4), e =
  // i/2, at d = 32db + 16((lane/16)%2) + 8(i%2); the result's element e is
  // then V[that row][32db + lane%32], and the rows of element e match the
  // keys of P^T's element e (C layout of S^T).  The swizzle depends on the
  // row mod 16, so kc adds 16 rows and db is the base XOR 32db.
  const int krow = 32 * kh + ln;
  const int kbase = krow * kDsRow + 16 * (hh ^ ds_swz_k(krow));
  int vbase;
  {
    const int i = lane & 15, e = i >> 1, s2 = (lane >> 4) & 1;
    const int r = 32 * kh + 4 * hh + (e & 3) + 8 * (e >> 2);
    vbase = r * kDsRow + 16 * (s2 ^ ds_swz_v(r)) + 8 * (i & 1);
  }

  const float c2 = a.scale_log2;
  const float lazy_raw = kLazyLog2 / c2;
  float m_run = kNegInf, l_run = 0.f;
  f32x16 acc[4];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[db][i] = 0.f;

  // ---- one tile, from stage Kc / Vc -------------------------------------------
  // after_reads() runs once this wave's fragment reads are issued
  // (Kc and Vc are not restrict: after_reads reloads the same stage)
  auto compute = [&](int t, const unsigned char* Kc, const unsigned char* Vc, auto&& after_reads)
                     __attribute__((always_inline)) {
    int kbo = kbase, vbo = vbase;
    asm volatile("" : "+v"(kbo), "+v"(vbo));
    // all of the tile's fragment reads first (K, then V^T)
    uint4 kr[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) kr[p] = *(const uint4*)(Kc + (kbo ^ (32 * p)));
    ds_v2i32 vr[4][2];
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int kc = 0; kc < 2; ++kc)
        vr[db][kc] = __builtin_amdgcn_ds_read_tr8_b64_v2i32((ds_lds_v2i32*)(Vc + ((vbo ^ (32 * db)) + 16 * kDsRow * kc)));
    __builtin_amdgcn_sched_barrier(0);
    after_reads();
    __builtin_amdgcn_sched_barrier(0);
    // S^T = K q^T, one MFMA per k-step; each step's VALU slot (the wave
    // issues while its MFMA runs) decodes the next K fragment and one V^T
    // fragment, so the V decode is off the softmax's path
    f32x16 sacc = {};
    uint4 vf[4][2];
    uint4 kfrag = fp8x8_to_bf16x8(kr[0].x, kr[0].y);
#pragma unroll
    for (int st = 0; st < 8; ++st) {
      sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(kfrag), qf[st], sacc, 0, 0, 0);
      if (st + 1 < 8) {
        const uint4 w = kr[(st + 1) >> 1];
        kfrag = ((st + 1) & 1) ? fp8x8_to_bf16x8(w.z, w.w) : fp8x8_to_bf16x8(w.x, w.y);
      }
      vf[st >> 1][st & 1] = fp8x8_to_bf16x8((uint32_t)vr[st >> 1][st & 1].x, (uint32_t)vr[st >> 1][st & 1].y);
      {   // decoded here, not next to its MFMA
        uint4& x = vf[st >> 1][st & 1];
        asm volatile("" : "+v"(x.x), "+v"(x.y), "+v"(x.z), "+v"(x.w));
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    // mask keys past the cache length and padding heads
    const int rem = n - t * 64 - 32 * kh;
    float sv[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) sv[i] = sacc[i];
    if (rem < 32 || !hvalid) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int off = 8 * (i >> 2) + 4 * hh + (i & 3);
        if (off >= rem || !hvalid) sv[i] = kNegInf;
      }
    }
    // online softmax (base 2), lazily moved reference
    float mt = kNegInf;
#pragma unroll
    for (int i = 0; i < 16; ++i) mt = fmaxf(mt, sv[i]);
    mt = xor32_max(mt);
    const bool moved = mt > m_run + lazy_raw;
    const float mref = moved ? mt : m_run;
    const float alpha = moved ? __builtin_amdgcn_exp2f((m_run - mref) * c2) : 1.f;
    m_run = mref;
    const float mc = (mref == kNegInf) ? 0.f : mref * c2;
    float pr[16];
#pragma unroll
    for (int i = 0; i < 8; ++i) pr[i] = __builtin_amdgcn_exp2f(fmaf(sv[i], c2, -mc));
    if (__ballot(moved) != 0ull) {
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[db][i] *= alpha;
    }
    auto pack8 = [](const float* x) __attribute__((always_inline)) {
      uint4 pk;
      pk.x = pack_bf16x2(x[0], x[1]);
      pk.y = pack_bf16x2(x[2], x[3]);
      pk.z = pack_bf16x2(x[4], x[5]);
      pk.w = pack_bf16x2(x[6], x[7]);
      return as_bf16x8(pk);
    };
    const bf16x8 pf0 = pack8(pr);
    __builtin_amdgcn_sched_barrier(0);
    // O^T += V^T P^T.  An MFMA that waits for the busy matrix pipe holds up
    // the SIMD's VALU issue, so each one is followed by about its own
    // duration of independent VALU work from this wave: the second half of
    // the probabilities, the token score (per-key max over this wave's heads
    // in registers; over the two head halves in LDS), the row sum.
    float w[8];
    acc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(vf[0][0]), pf0, acc[0], 0, 0, 0);
    pr[8] = __builtin_amdgcn_exp2f(fmaf(sv[8], c2, -mc));
    pr[9] = __builtin_amdgcn_exp2f(fmaf(sv[9], c2, -mc));
    w[0] = colmax16_swap(sv[0], sv[8]);
    w[1] = colmax16_swap(sv[1], sv[9]);
    __builtin_amdgcn_sched_barrier(0);
    acc[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(vf[1][0]), pf0, acc[1], 0, 0, 0);
    pr[10] = __builtin_amdgcn_exp2f(fmaf(sv[10], c2, -mc));
    pr[11] = __builtin_amdgcn_exp2f(fmaf(sv[11], c2, -mc));
    w[2] = colmax16_swap(sv[2], sv[10]);
    w[3] = colmax16_swap(sv[3], sv[11]);
    __builtin_amdgcn_sched_barrier(0);
    acc[2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(vf[2][0]), pf0, acc[2], 0, 0, 0);
    pr[12] = __builtin_amdgcn_exp2f(fmaf(sv[12], c2, -mc));
    pr[13] = __builtin_amdgcn_exp2f(fmaf(sv[13], c2, -mc));
    w[4] = colmax16_swap(sv[4], sv[12]);
    w[5] = colmax16_swap(sv[5], sv[13]);
    __builtin_amdgcn_sched_barrier(0);
    acc[3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(vf[3][0]), pf0, acc[3], 0, 0, 0);
    pr[14] = __builtin_amdgcn_exp2f(fmaf(sv[14], c2, -mc));
    pr[15] = __builtin_amdgcn_exp2f(fmaf(sv[15], c2, -mc));
    w[6] = colmax16_swap(sv[6], sv[14]);
    w[7] = colmax16_swap(sv[7], sv[15]);
    const bf16x8 pf1 = pack8(pr + 8);
    __builtin_amdgcn_sched_barrier(0);
    acc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(vf[0][1]), pf1, acc[0], 0, 0, 0);
    const f32x2 m2 = colmax16_dpp(w);
    __builtin_amdgcn_sched_barrier(0);
    acc[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(vf[1][1]), pf1, acc[1], 0, 0, 0);
    {
      const int R = lane >> 4, j = lane & 15;
      const int r0 = 16 * (R & 1) + 8 * (j >> 3) + 4 * (R >> 1) + 2 * ((j >> 2) & 1);
      if ((j & 3) == 0) *(f32x2*)&red[t & 1][hb][32 * kh + r0] = m2;
    }
    float ps0 = 0.f, ps1 = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) ps0 += pr[i];
    __builtin_amdgcn_sched_barrier(0);
    acc[2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(vf[2][1]), pf1, acc[2], 0, 0, 0);
#pragma unroll
    for (int i = 8; i < 16; ++i) ps1 += pr[i];
    l_run = fmaf(l_run, alpha, ps0 + ps1);
    __builtin_amdgcn_sched_barrier(0);
    acc[3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(vf[3][1]), pf1, acc[3], 0, 0, 0);
  };

  // token scores of tile t (keys t*64 + lane), from red[t & 1]; wave 0
  auto emit_scores = [&](int t) __attribute__((always_inline)) {
    if (wave == 0) {
      const int j = t * 64 + lane;
      const float v = fmaxf(red[t & 1][0][lane], red[t & 1][1][lane]);
      if (j < a.Nmax) a.scores[(int64_t)b * a.sc_sb + j] = (j < n) ? v * a.logit_scale : kNegInf;
    }
  };

  // ---- tile pipeline.  Iteration t waits for its own loads of tile t (the
  // three tiles after it may still be in flight), then the barrier: tile t
  // has landed for every wave.  Each wave reads its fragments of tile t; a
  // second barrier (every wave's reads returned) frees the stage for the
  // loads of tile t+4.  The main loop runs only while every iteration of a
  // group of four has a tile four ahead, so its loads and waits are
  // unconditional: the compiler's own wait before a stage's reads then sees
  // that stage's last load followed by the three others on every path, and
  // the barrier's vmcnt(12) covers it.  The last (at most seven) tiles run
  // in a tail without a back edge. ----------------------------------------------
  auto step = [&](auto full_tag, int t, unsigned char* Kc, unsigned char* Vc) __attribute__((always_inline)) {
    constexpr bool FULL = decltype(full_tag)::value;
    if (FULL || t + 3 < t1) ds_tile_barrier<12>();
    else if (t + 2 < t1) ds_tile_barrier<8>();
    else if (t + 1 < t1) ds_tile_barrier<4>();
    else ds_tile_barrier<0>();
    if (t > t0) emit_scores(t - 1);
    compute(t, Kc, Vc, [&]() __attribute__((always_inline)) {
      if (FULL || t + 4 < t1) {
        ds_reads_barrier();
        load_tile(t + 4, Kc, Vc);
      }
    });
  };
  using Full = std::integral_constant<bool, true>;
  using Tail = std::integral_constant<bool, false>;
  int t = t0;
  if (t0 + 7 < t1) {
    load_tile(t0, K0, V0);
    load_tile(t0 + 1, K1, V1);
    load_tile(t0 + 2, K2, V2);
    load_tile(t0 + 3, K3, V3);
    do {
      step(Full{}, t, K0, V0);
      step(Full{}, t + 1, K1, V1);
      step(Full{}, t + 2, K2, V2);
      step(Full{}, t + 3, K3, V3);
      t += 4;
    } while (t + 7 < t1);
  } else {
    if (t0 < t1) load_tile(t0, K0, V0);
    if (t0 + 1 < t1) load_tile(t0 + 1, K1, V1);
    if (t0 + 2 < t1) load_tile(t0 + 2, K2, V2);
    if (t0 + 3 < t1) load_tile(t0 + 3, K3, V3);
  }
  // tail: tiles t .. t1-1 (at most seven), stages continuing from 0
  if (t < t1) step(Tail{}, t, K0, V0);
  if (t + 1 < t1) step(Tail{}, t + 1, K1, V1);
  if (t + 2 < t1) step(Tail{}, t + 2, K2, V2);
  if (t + 3 < t1) step(Tail{}, t + 3, K3, V3);
  if (t + 4 < t1) step(Tail{}, t + 4, K0, V0);
  if (t + 5 < t1) step(Tail{}, t + 5, K1, V1);
  if (t + 6 < t1) step(Tail{}, t + 6, K2, V2);
  ds_tile_barrier<0>();
  if (t0 < t1) emit_scores(t1 - 1);
  // keys past the valid length: token scores are -inf (the workgroups of the
  // last split cover the tail of the score row)
  if (s == a.nsplit - 1) {
    for (int j = ntiles * 64 + tid; j < a.Nmax; j += 256) a.scores[(int64_t)b * a.sc_sb + j] = kNegInf;
  }

  // ---- merge the two key halves' (m, l, O) of each head half, then write the
  // workgroup's partial.  The ring is free (every load landed, every read is
  // done): head half 0 takes K0 and K1 for O, head half 1 V0 and V1, both K2
  // for m and l.
  float* oa = (float*)(hb ? V0 : K0);
  float* ob = (float*)(hb ? V1 : K1);
  float* ml = (float*)K2 + hb * 128;
  if (kh == 1) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      oa[i * 64 + lane] = acc[0][i];
      oa[(16 + i) * 64 + lane] = acc[1][i];
      ob[i * 64 + lane] = acc[2][i];
      ob[(16 + i) * 64 + lane] = acc[3][i];
    }
    ml[lane] = m_run;
    ml[64 + lane] = l_run;
  }
  ds_tile_barrier<0>();
  if (kh == 0 && hvalid) {
    const float m1 = ml[lane], l1 = ml[64 + lane];
    const float M = fmaxf(m_run, m1);
    const float w0 = (m_run == kNegInf) ? 0.f : __builtin_amdgcn_exp2f((m_run - M) * c2);
    const float w1 = (m1 == kNegInf) ? 0.f : __builtin_amdgcn_exp2f((m1 - M) * c2);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      acc[0][i] = acc[0][i] * w0 + oa[i * 64 + lane] * w1;
      acc[1][i] = acc[1][i] * w0 + oa[(16 + i) * 64 + lane] * w1;
      acc[2][i] = acc[2][i] * w0 + ob[i * 64 + lane] * w1;
      acc[3][i] = acc[3][i] * w0 + ob[(16 + i) * 64 + lane] * w1;
    }
    const float lm = l_run * w0 + l1 * w1;
    const float lsum = lm + __shfl_xor(lm, 32);
    const int64_t pidx = ((int64_t)(layer * a.B + b) * a.nsplit + s) * a.Hq + head;
    float* po = a.part_o + pidx * kDsD;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const int d = db * 32 + 8 * i4 + 4 * hh;
        const float4 v4 = {acc[db][4 * i4], acc[db][4 * i4 + 1], acc[db][4 * i4 + 2], acc[db][4 * i4 + 3]};
        *(float4*)(po + d) = v4;
      }
    if (hh == 0) { a.part_ml[pidx * 2] = M; a.part_ml[pidx * 2 + 1] = lsum; }
  }
}

}  // namespace

bool decode_split_fp8_supported(int D, const DecArgs& a) {
  const uintptr_t kp = (uintptr_t)a.k, vp = (uintptr_t)a.v;
  return D == kDsD && a.nlayer == 1 && a.k_sl == 0 && a.v_sl == 0 && a.sc_sl == 0 && (kp % 16) == 0 && (vp % 16) == 0 && a.k_sb % 16 == 0 && a.v_sb % 16 == 0 &&
         a.k_st % 16 == 0 && a.v_st % 16 == 0 && a.k_st >= kDsD && a.v_st >= kDsD &&
         64 * a.k_st < ((int64_t)1 << 32) && 64 * a.v_st < ((int64_t)1 << 32);
}

hipError_t launch_decode_split_fp8(const DecArgs& a, hipStream_t s) {
  const unsigned grid = (unsigned)(a.nlayer * a.B * a.nsplit);
  hipLaunchKernelGGL(decode_split_fp8_kernel, dim3(grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace hys
