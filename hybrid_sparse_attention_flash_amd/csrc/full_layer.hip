// The HySparse full layer for bf16 Q/K/V on gfx950: exact causal attention
// that also emits the block scores the sparse layers select from.
//
// What it computes (QbitAI HySparse article, method section; TechWalker
// HySparse write-up, paragraph on the modified FlashAttention kernel): for
// every query row, softmax(q K^T * scale) V over the keys at or before its
// position, its log-sum-exp, and, with scores on, for every 64-key block c the
// maximum over the block's visible keys of the scaled logit, reduced over the
// query heads of the row's KV group (blocks past the query's own hold -inf).
// The tiled engine's M_FULL / M_FULL_BLOCK modes compute the same for fp32
// and fp8 inputs and for head groups this kernel does not take.
//
// Design:
//  * A workgroup (8 waves, one per CU) owns BQ = 256 / G queries x the G
//    heads of one KV group, row r = query r / G, head r % G; each wave owns
//    32 consecutive rows, the N of v_mfma_f32_32x32x16_bf16.  It walks the
//    64-key tiles 0 .. its last query's block.
//  * Key tiles go HBM -> LDS with global_load_lds_dwordx4 (each lane fetches
//    any 16 bytes; the 64 lanes of one instruction fill 1 KiB of LDS in lane
//    order): no staging registers and no VALU work.  Three LDS stages: the
//    loads of tiles n+1 and n+2 are in flight while tile n is computed (one
//    tile of lead left their latency exposed at every barrier); one barrier a
//    tile.
//  * K and V sit in LDS row-major, [64 keys][D], the 16-byte chunks of each
//    row XOR-swizzled so the fragment reads below are free of bank conflicts.
//    S^T = K Q^T takes K fragments (A) with ds_read_b128 and Q (B) from
//    registers; each lane then holds one row's logits for 32 of the 64 keys,
//    so the row maximum needs one cross-lane exchange.  O^T = V^T P^T takes
//    the V^T fragments (A) from row-major V with ds_read_b64_tr_b16 and P^T
//    (B) straight from the logit registers.
//  * Online softmax in the base-2 domain on raw dot products with a lazily
//    moved reference (the engine's rule); the block score is the row's tile
//    maximum, reduced over a query's heads between adjacent lanes.
//
// v_mfma_f32_32x32x16_bf16 lane layout (wave64, lane l = 32h + n): lane l holds
// A[m = l%32][k = 8h + j], B[k = 8h + j][n = l%32] (j = 0..7) and
// C[m = 8(i/4) + 4h + i%4][n = l%32] (i = 0..15).
#include "common.h"
#include "kernels.h"
#include <type_traits>

namespace hys {
namespace {

typedef short fl_v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void fl_lds_void;
typedef __attribute__((address_space(3))) fl_v4i16 fl_lds_v4i16;

constexpr int kFlRows = kFullLayerRows;         // rows per workgroup
constexpr int kFlWaves = kFlRows / 32;          // waves per workgroup
static_assert(kFlWaves == 8, "the load placement assumes 8 waves");

template <int D> struct FGeo {
  static constexpr int ROWB = 2 * D;            // bytes per key row
  static constexpr int CPR = D / 8;             // 16-byte chunks per row
  static constexpr int RPI = 1024 / ROWB;       // rows filled by one load instruction
  static constexpr int NU = 64 / (kFlWaves * RPI);   // load instructions per wave, operand and tile
  static constexpr int TILEB = 64 * ROWB;       // bytes of one operand tile
  static constexpr int NQC = D / 16;            // k-steps of S^T
  static constexpr int NDB = D / 32;            // 32-wide d blocks of O^T
};

// chunk c of key row r is stored at chunk c ^ swz(r).  K: the 32 rows one
// ds_read_b128 addresses (one chunk each) fall in distinct banks on 32- and
// 64-bank LDS.  V: the transposing reads' four-row slices likewise.  Both
// depend on the row mod 32 only (rows ln and ln + 32 share a swizzle).
template <int D> __device__ __forceinline__ int fswz_k(int r) { return D == 128 ? (r & 15) : ((r ^ ((r >> 3) & 3)) & 7); }
template <int D> __device__ __forceinline__ int fswz_v(int r) { return D == 128 ? (5 * (r & 3)) & 15 : 2 * (r & 3); }

// this wave's LDS reads and writes are done and at most PENDING of its LDS
// loads are still in flight (loads complete in issue order, so these are the
// newest); then the workgroup barrier (a compiler barrier for memory as well)
template <int PENDING>
__device__ __forceinline__ void fl_tile_barrier() {
  static_assert(PENDING >= 0 && PENDING < 16, "vmcnt field");
  __builtin_amdgcn_s_waitcnt(0x0070 | PENDING);   // vmcnt(PENDING) lgkmcnt(0)
  asm volatile("s_barrier" ::: "memory");
}

template <int D, bool SCORES>
__global__ __launch_bounds__(kFlRows * 2, 2) void full_layer_kernel(const AttnArgs a) {
  using P = FGeo<D>;
  // three stages (tile n is computed while tiles n+1 and n+2 load), each
  // operand and stage its own array: every LDS access below names one of
  // them statically (the tile loop is unrolled by three), which is what lets
  // the compiler tell the loads into one stage from the reads of another and
  // keep the loads in flight across whole tiles
  __shared__ __attribute__((aligned(1024))) unsigned char K0[P::TILEB];
  __shared__ __attribute__((aligned(1024))) unsigned char K1[P::TILEB];
  __shared__ __attribute__((aligned(1024))) unsigned char K2[P::TILEB];
  __shared__ __attribute__((aligned(1024))) unsigned char V0[P::TILEB];
  __shared__ __attribute__((aligned(1024))) unsigned char V1[P::TILEB];
  __shared__ __attribute__((aligned(1024))) unsigned char V2[P::TILEB];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hh = lane >> 5, ln = lane & 31;
  if ((int)blockIdx.x >= a.grid_used) return;

  // ---- work item: KV group fastest (the 8 XCDs take the workgroups round
  // robin, so each XCD's L2 serves few KV heads), longest query tiles first --
  const int g = (int)blockIdx.x % a.Hkv;
  const int rest = (int)blockIdx.x / a.Hkv;
  const int b = rest % a.B;
  const int qt = a.ntq - 1 - rest / a.B;
  const int q0 = qt * a.BQ;
  const int nq = min(a.BQ, a.Lq - q0);
  const int HC = a.HC;
  // absolute position of the last query (row r of the call is q_off + r)
  const int qa_last = q0 + nq - 1 + a.q_off;

  // ---- this lane's row ---------------------------------------------------------
  const int r = wave * 32 + ln;
  const int qi = r / HC;
  const int qpos = q0 + qi;
  const int head = g * a.G + (r - qi * HC);
  const bool valid = qi < nq;
  const int qa = qpos + a.q_off;

  // ---- Q fragments (B of S^T): q[row][16c + 8hh .. +7] ----------------------
  const uint16_t* qbase = (const uint16_t*)a.q + (int64_t)b * a.q_sb;
  bf16x8 qf[P::NQC];
  {
    const uint16_t* qr = qbase + (valid ? (int64_t)qpos * a.q_st + (int64_t)head * a.q_sh : 0);
#pragma unroll
    for (int c = 0; c < P::NQC; ++c) {
      const uint4 x = *(const uint4*)(qr + 16 * c + 8 * hh);
      const uint4 z = {0u, 0u, 0u, 0u};
      qf[c] = as_bf16x8(valid ? x : z);
    }
  }

  // ---- tiles 0 .. the last query's block ---------------------------------------
  const int ntiles = qa_last / 64 + 1;
  const int jlast = a.Lk - 1;
  const uint16_t* kb = (const uint16_t*)a.k + (int64_t)b * a.k_sb + (int64_t)g * a.k_sh;
  const uint16_t* vb = (const uint16_t*)a.v + (int64_t)b * a.v_sb + (int64_t)g * a.v_sh;
  // instruction u of this wave fills tile rows (8u + wave) * RPI + (0..RPI-1);
  // the swizzles depend on the row mod 16 (D = 128, where 8 * RPI = 32) and
  // D = 64 takes one instruction, so the chunk a lane fetches is the same
  // for every u: one lane offset from a tile's first row, the rest of each
  // address scalar
  const int drow0 = wave * P::RPI + lane / P::CPR;
  const uint32_t kstb = (uint32_t)a.k_st * 2u, vstb = (uint32_t)a.v_st * 2u;
  const uint32_t chunk_k = (uint32_t)(((lane % P::CPR) ^ fswz_k<D>(drow0)) * 16);
  const uint32_t chunk_v = (uint32_t)(((lane % P::CPR) ^ fswz_v<D>(drow0)) * 16);
  const uint32_t lane_k = (uint32_t)drow0 * kstb + chunk_k;
  const uint32_t lane_v = (uint32_t)drow0 * vstb + chunk_v;
  // (64 rows of K or V span less than 2^32 bytes: checked at launch)
  auto load_tile = [&](int j0, unsigned char* Kd, unsigned char* Vd, uint32_t lk, uint32_t lv, const uint16_t* Kg,
                       const uint16_t* Vg) __attribute__((always_inline)) {
    const char* kt = (const char*)Kg + (int64_t)j0 * a.k_st * 2;
    const char* vt = (const char*)Vg + (int64_t)j0 * a.v_st * 2;
    if (j0 + 63 <= jlast) {
      // scalar row base per instruction + the lane's fixed offset: the two
      // offset registers stay live through the loop, so no LDS read result is
      // ever given a register an in-flight load still names
#pragma unroll
      for (int u = 0; u < P::NU; ++u) {
        const char* ktu = kt + (int64_t)(kFlWaves * P::RPI * u) * a.k_st * 2;
        const char* vtu = vt + (int64_t)(kFlWaves * P::RPI * u) * a.v_st * 2;
        __builtin_amdgcn_global_load_lds((const void*)(ktu + lk), (fl_lds_void*)(Kd + (kFlWaves * u + wave) * 1024), 16, 0, 0);
        __builtin_amdgcn_global_load_lds((const void*)(vtu + lv), (fl_lds_void*)(Vd + (kFlWaves * u + wave) * 1024), 16, 0, 0);
      }
    } else {
      // last tile of the keys: slots past the last key repeat the last key's
      // row (their logits are masked, so their probabilities are exactly 0)
      const int rmax = jlast - j0;
#pragma unroll
      for (int u = 0; u < P::NU; ++u) {
        const uint32_t rr = (uint32_t)min(drow0 + kFlWaves * P::RPI * u, rmax);
        __builtin_amdgcn_global_load_lds((const void*)(kt + (rr * kstb + chunk_k)), (fl_lds_void*)(Kd + (kFlWaves * u + wave) * 1024), 16, 0, 0);
        __builtin_amdgcn_global_load_lds((const void*)(vt + (rr * vstb + chunk_v)), (fl_lds_void*)(Vd + (kFlWaves * u + wave) * 1024), 16, 0, 0);
      }
    }
  };

  // per-lane LDS byte offsets inside a tile.  K, k-step c, key ln (+32):
  // row ln, chunk 2c + hh, stored at (2c + hh) ^ swz_k(ln); the swizzle only
  // flips chunk bits, so step c is the base XOR 32c.  V^T, d block db, k-step
  // kc: the lane's 16-lane slice (i = lane % 16, slice bit s = (lane / 16) % 2)
  // addresses rows 4hh + i/4 (+16kc, +8) at d = 32db + 16s + 4(i%4); the
  // swizzle flips only the d-block bits and those below, so block db is the
  // base XOR 64db.
  const int kbase_off = ln * P::ROWB + ((hh ^ fswz_k<D>(ln)) * 16);
  int vbase_off;
  {
    const int i = lane & 15, s = (lane >> 4) & 1;
    const int vr = 4 * hh + (i >> 2), sv = fswz_v<D>(vr);
    const int x = 2 * s + ((i >> 1) & 1);            // chunk among the d block's four
    vbase_off = vr * P::ROWB + 64 * (sv >> 2) + 16 * (x ^ (sv & 3)) + 8 * (i & 1);
  }

  // ---- softmax state -------------------------------------------------------
  const float c2 = a.scale_log2;
  const float lazy_raw = kLazyLog2 / c2;
  float m_run = kNegInf, l_run = 0.f;
  f32x16 acc[P::NDB];
#pragma unroll
  for (int db = 0; db < P::NDB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[db][i] = 0.f;
  // block scores of this lane's query: a scalar base and a 32-bit lane offset
  // (a KV group's score matrix spans less than 2^32 entries: checked at launch)
  float* sc_base = nullptr;
  if (SCORES) sc_base = a.scores + (int64_t)g * a.sc_sg + (int64_t)b * a.sc_sb;
  const uint32_t sc_off = valid ? (uint32_t)qpos * (uint32_t)a.sc_sr : 0u;
  const bool sc_lane = SCORES && valid && hh == 0 && (ln % HC) == 0;

  // ---- one tile ---------------------------------------------------------------
  // Kc/Vc: the tile being computed; Kn/Vn: the stage tile n+2 is loaded into
  // (the one tile n-1 was read from); Kg/Vg: the K and V rows in global
  // memory.  The barrier at the end waits for tile n+1's loads only, so each
  // tile's loads have two tiles of compute to land in.
  auto step = [&](auto mask_tag, int n, const unsigned char* __restrict__ Kc, const unsigned char* __restrict__ Vc,
                  unsigned char* __restrict__ Kn, unsigned char* __restrict__ Vn, const uint16_t* __restrict__ Kg,
                  const uint16_t* __restrict__ Vg) __attribute__((always_inline)) {
    // the per-step fragment offsets are a few XORs of these bases;
    // recomputing them each tile keeps them out of the register budget the
    // loop would otherwise hold them in
    int kbo = kbase_off, vbo = vbase_off;
    asm volatile("" : "+v"(kbo), "+v"(vbo));
    const bool more = n + 2 < ntiles;
    if (more) load_tile(64 * (n + 2), Kn, Vn, lane_k, lane_v, Kg, Vg);
    const int j0 = 64 * n;
    // MASK: the tile may hold keys past some row's position (the last one or
    // two tiles of the workgroup); other tiles are whole for every row.  (A
    // wave none of whose rows sees a tile, possible only in the last tile when
    // the rows start mid-block, runs it anyway: every row is off, so it adds
    // nothing and its block scores come out -inf.)
    constexpr bool MASK = decltype(mask_tag)::value;
    {
      const bool row_on = MASK ? (valid && j0 <= qa) : valid;
      // The tile runs as two 32-key halves h (keys j0 + 32h ..), each its own
      // online-softmax step.  A wave issues in order, so the overlap of
      // matrix and vector work is laid out by hand, in chunks the compiler
      // may not reorder across (sched_barrier): the softmax of half 0 runs
      // between the S MFMAs of half 1, that of half 1 between the PV MFMAs of
      // half 0, the block-score reduction between those of half 1.  The
      // reference moves branch-free (alpha = 1 unless it moves); only the
      // rare rescale of O is a branch, between the PV MFMAs of the halves.
      f32x16 s[2];
      const f32x16 zero16 = {};
      // K fragment t: half t / NQC (rows 32h + ln), k-step t % NQC
      constexpr int NT = 2 * P::NQC;
      auto kfrag = [&](int t) __attribute__((always_inline)) {
        return *(const uint4*)(Kc + (kbo ^ (32 * (t % P::NQC))) + (t / P::NQC) * 32 * P::ROWB);
      };
      // V^T fragments of d block db, k-step kc: keys 16kc + 4hh + (0..3) (lo)
      // and 16kc + 8 + 4hh + (0..3) (hi) at d = 32db + ln
      auto vfrag = [&](int db, int kc) __attribute__((always_inline)) {
        const unsigned char* vr = Vc + (vbo ^ (64 * db)) + (16 * kc) * P::ROWB;
        const fl_v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((fl_lds_v4i16*)vr);
        const fl_v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((fl_lds_v4i16*)(vr + 8 * P::ROWB));
        const uint2 l2 = __builtin_bit_cast(uint2, lo), h2 = __builtin_bit_cast(uint2, hi);
        return make_uint4(l2.x, l2.y, h2.x, h2.y);
      };
      // softmax of half h, in parts: head (mask, maximum, reference), the
      // probabilities of elements [e0, e1), tail (row sum, P^T fragments)
      float mt_h[2], alpha_h[2], mc_h[2], ps_h[2];
      bool need_h[2];
      auto soft_head = [&](int h) __attribute__((always_inline)) {
        f32x16& x = s[h];
        if (MASK) {
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int key = j0 + 32 * h + 8 * (i >> 2) + 4 * hh + (i & 3);
            x[i] = (row_on & (key <= qa)) ? x[i] : kNegInf;
          }
        }
        float m4[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
          m4[e] = fmax_nc(fmax_nc(x[4 * e], x[4 * e + 1]), fmax_nc(x[4 * e + 2], x[4 * e + 3]));
        float mt = xor32_max(fmax_nc(fmax_nc(m4[0], m4[1]), fmax_nc(m4[2], m4[3])));
        if (!row_on) mt = kNegInf;
        mt_h[h] = mt;
        const bool need = mt > m_run + lazy_raw;
        const float mref = need ? mt : m_run;
        // (exp2 of 0 when the reference stays; -inf, giving 0, when it moves
        // off -inf; computed unconditionally so no branch splits the code)
        alpha_h[h] = __builtin_amdgcn_exp2f(need ? (m_run - mref) * c2 : 0.f);
        need_h[h] = need;
        m_run = mref;
        float mc = mref * c2;
        mc = (mref == kNegInf) ? 0.f : mc;
        mc_h[h] = row_on ? mc : __builtin_huge_valf();
        ps_h[h] = 0.f;
      };
      auto soft_exp = [&](int h, int e0, int e1) __attribute__((always_inline)) {
#pragma unroll
        for (int e = e0; e < e1; ++e) {
          s[h][e] = __builtin_amdgcn_exp2f(fmaf(s[h][e], c2, -mc_h[h]));
          ps_h[h] += s[h][e];
        }
      };
      auto soft_tail = [&](int h, bf16x8 (&pf)[2]) __attribute__((always_inline)) -> bool {
        l_run = fmaf(l_run, alpha_h[h], ps_h[h]);
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          uint4 pk;
          pk.x = pack_bf16x2(s[h][8 * q + 0], s[h][8 * q + 1]);
          pk.y = pack_bf16x2(s[h][8 * q + 2], s[h][8 * q + 3]);
          pk.z = pack_bf16x2(s[h][8 * q + 4], s[h][8 * q + 5]);
          pk.w = pack_bf16x2(s[h][8 * q + 6], s[h][8 * q + 7]);
          pf[q] = as_bf16x8(pk);
        }
        return __ballot(need_h[h]) != 0ull;
      };
      // the 16 elements of a half exponentiated in NS chunks: chunk k covers
      // [16k / NS, 16(k + 1) / NS)
      auto soft_chunk = [&](int h, int k, int ns) __attribute__((always_inline)) {
        soft_exp(h, 16 * k / ns, 16 * (k + 1) / ns);
      };
      constexpr int NSA = P::NQC - 2;       // half 0: after the 3rd S MFMA of half 1
      constexpr int NSB = 2 * P::NDB - 1;   // half 1: after the 2nd PV MFMA of half 0

      // ---- S^T = K Q^T; half 0's softmax between half 1's last 6 MFMAs ----
      uint4 kf[NT];
      kf[0] = kfrag(0);
      kf[1] = kfrag(1);
      kf[2] = kfrag(2);
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        if (t + 3 < NT) kf[t + 3] = kfrag(t + 3);
        const int h = t / P::NQC, c = t % P::NQC;
        s[h] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(kf[t]), qf[c], c == 0 ? zero16 : s[h], 0, 0, 0);
        if (t == P::NQC + 1) soft_head(0);            // S of half 0 has landed by now
        if (t >= P::NQC + 2) soft_chunk(0, t - P::NQC - 2, NSA);
        __builtin_amdgcn_sched_barrier(0);
      }
      bf16x8 pf0[2], pf1[2];
      const bool moved0 = soft_tail(0, pf0);
      // the probabilities are pinned ahead of the rescale branch (the
      // compiler would otherwise sink them past it)
      asm volatile("" : "+v"(pf0[0]), "+v"(pf0[1]), "+v"(l_run));
      if (moved0) {
#pragma unroll
        for (int db = 0; db < P::NDB; ++db) acc[db] *= alpha_h[0];
      }

      // ---- O^T += V^T P^T_0 (k-steps 0, 1); half 1's softmax between -------
      {
        uint4 vf[2][2];
        vf[0][0] = vfrag(0, 0);
        vf[0][1] = vfrag(0, 1);
#pragma unroll
        for (int i = 0; i < 2 * P::NDB; ++i) {
          const int db = i / 2, q = i % 2;
          if (q == 0 && db + 1 < P::NDB) {
            vf[(db + 1) & 1][0] = vfrag(db + 1, 0);
            vf[(db + 1) & 1][1] = vfrag(db + 1, 1);
          }
          acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(vf[db & 1][q]), pf0[q], acc[db], 0, 0, 0);
          if (i == 0) soft_head(1);
          if (i >= 1) soft_chunk(1, i - 1, NSB);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      const bool moved1 = soft_tail(1, pf1);
      asm volatile("" : "+v"(pf1[0]), "+v"(pf1[1]), "+v"(l_run));
      if (moved1) {
#pragma unroll
        for (int db = 0; db < P::NDB; ++db) acc[db] *= alpha_h[1];
      }

      // ---- O^T += V^T P^T_1 (k-steps 2, 3); the block score between ----------
      // (the row's tile maximum reduced over the query's HC adjacent lanes, HC
      // in 1, 2, 4, 8, 16, 32: every step taken and selected, no branch)
      float gm = fmax_nc(mt_h[0], mt_h[1]);
      auto gstep = [&](int k) __attribute__((always_inline)) {
        float t;
        if (k == 0) t = __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, gm), 0xB1, 0xF, 0xF, false));
        else if (k == 1) t = __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, gm), 0x4E, 0xF, 0xF, false));
        else if (k == 2) t = __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, gm), 0x141, 0xF, 0xF, false));
        else if (k == 3) t = __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, gm), 0x140, 0xF, 0xF, false));
        else t = xor16_max(gm);
        t = fmax_nc(gm, t);
        gm = HC >= (2 << k) ? t : gm;
      };
      {
        uint4 vf[2][2];
        vf[0][0] = vfrag(0, 2);
        vf[0][1] = vfrag(0, 3);
#pragma unroll
        for (int i = 0; i < 2 * P::NDB; ++i) {
          const int db = i / 2, q = i % 2;
          if (q == 0 && db + 1 < P::NDB) {
            vf[(db + 1) & 1][0] = vfrag(db + 1, 2);
            vf[(db + 1) & 1][1] = vfrag(db + 1, 3);
          }
          acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(vf[db & 1][q]), pf1[q], acc[db], 0, 0, 0);
          if (SCORES && i < 5) gstep(i);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      if (SCORES && sc_lane) sc_base[sc_off + n] = gm * a.logit_scale;
    }
    if (more) fl_tile_barrier<2 * P::NU>();
    else fl_tile_barrier<0>();
  };

  // tiles 0 .. nfull-1 are whole for every row of the workgroup (their last
  // key precedes its first query); the rest need the causal mask
  const int nfull = min((q0 + a.q_off + 1) / 64, ntiles);
  load_tile(0, K0, V0, lane_k, lane_v, kb, vb);
  if (ntiles > 1) {
    load_tile(64, K1, V1, lane_k, lane_v, kb, vb);
    fl_tile_barrier<2 * P::NU>();
  } else {
    fl_tile_barrier<0>();
  }
  // tile n is read from stage n % 3; step n loads tile n + 2 into stage
  // (n + 2) % 3.  The main loop takes three mask-free tiles per trip; the
  // rest go through a switch on the stage (a handful of tiles per workgroup).
  auto one = [&](auto mask_tag, int n) __attribute__((always_inline)) {
    switch (n % 3) {
      case 0: step(mask_tag, n, K0, V0, K2, V2, kb, vb); break;
      case 1: step(mask_tag, n, K1, V1, K0, V0, kb, vb); break;
      default: step(mask_tag, n, K2, V2, K1, V1, kb, vb); break;
    }
  };
  int n = 0;
  for (; n + 2 < nfull; n += 3) {
    step(std::false_type{}, n, K0, V0, K2, V2, kb, vb);
    step(std::false_type{}, n + 1, K1, V1, K0, V0, kb, vb);
    step(std::false_type{}, n + 2, K2, V2, K1, V1, kb, vb);
  }
  for (; n < nfull; ++n) one(std::false_type{}, n);
  for (; n < ntiles; ++n) one(std::true_type{}, n);

  // -inf for the blocks after each query's own
  if (SCORES) {
    float* sc = a.scores + (int64_t)g * a.sc_sg + (int64_t)b * a.sc_sb;
    const int ncol = a.nblk - ntiles;
    if (ncol > 0)
      for (int e = tid; e < nq * ncol; e += kFlRows * 2) {
        const int t = e / ncol, c = ntiles + (e - t * ncol);
        sc[(int64_t)(q0 + t) * a.sc_sr + c] = kNegInf;
      }
  }

  // ---- epilogue ----------------------------------------------------------------
  const float lsum = l_run + __shfl_xor(l_run, 32);
  const bool live = m_run != kNegInf;
  if (!valid) return;
  const float inv = live ? a.v_scale / lsum : 0.f;
  if (a.lse && hh == 0)
    a.lse[((int64_t)b * a.Hq + head) * a.Lq + qpos] = live ? (m_run * a.logit_scale + __logf(lsum)) : kNegInf;
  const int64_t ro = (int64_t)b * a.o_sb + (int64_t)qpos * a.o_st + (int64_t)head * a.o_sh;
#pragma unroll
  for (int db = 0; db < P::NDB; ++db)
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      const int d = db * 32 + 8 * i4 + 4 * hh;
      const float r0 = acc[db][4 * i4] * inv, r1 = acc[db][4 * i4 + 1] * inv;
      const float r2 = acc[db][4 * i4 + 2] * inv, r3 = acc[db][4 * i4 + 3] * inv;
      if (a.o_f32) {
        *(float4*)((float*)a.o + ro + d) = make_float4(r0, r1, r2, r3);
      } else {
        *(uint2*)((uint16_t*)a.o + ro + d) = make_uint2(pack_bf16x2(r0, r1), pack_bf16x2(r2, r3));
      }
    }
}

}  // namespace

bool full_layer_supported(int D, const AttnArgs& a, bool scores) {
  if (D != 64 && D != 128) return false;
  if (a.HC != a.G || a.nhc != 1 || a.BQ != kFlRows / a.G || a.BQ < 1) return false;
  // block scores reduce a query's heads between adjacent lanes of one wave,
  // and a lane addresses its query's scores with a 32-bit offset
  if (scores && (a.HC > 32 || 32 % a.HC != 0)) return false;
  if (scores && (int64_t)a.Lq * a.sc_sr >= (1ll << 32)) return false;
  // 64 rows of K or V are addressed with 32-bit offsets
  if (64 * a.k_st >= (1ll << 31) || 64 * a.v_st >= (1ll << 31)) return false;
  return true;
}

hipError_t launch_full_layer(int D, const AttnArgs& a, bool scores, int grid, hipStream_t s) {
  if (!full_layer_supported(D, a, scores)) return hipErrorInvalidValue;
  if (D == 64) {
    if (scores) hipLaunchKernelGGL((full_layer_kernel<64, true>), dim3(grid), dim3(2 * kFlRows), 0, s, a);
    else hipLaunchKernelGGL((full_layer_kernel<64, false>), dim3(grid), dim3(2 * kFlRows), 0, s, a);
  } else {
    if (scores) hipLaunchKernelGGL((full_layer_kernel<128, true>), dim3(grid), dim3(2 * kFlRows), 0, s, a);
    else hipLaunchKernelGGL((full_layer_kernel<128, false>), dim3(grid), dim3(2 * kFlRows), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace hys
