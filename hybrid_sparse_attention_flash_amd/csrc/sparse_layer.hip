// One-pass HySparse sparse layer for bf16 Q/K/V on gfx950: the key blocks each
// query selected from the shared K/V, then the layer's own sliding window,
// merged by the sigmoid gate.
//
// What it computes (QbitAI HySparse article, method section; TechWalker
// HySparse write-up, sparse-layer paragraph): for every query row, a causal
// softmax attention over the keys of the blocks its query selected, a second
// softmax attention over the last `window` positions of the layer's own K/V,
// and o = g * o_sparse + (1 - g) * o_window with g = sigmoid(<q, w_h> + b_h);
// a row whose selection sees no key gets o_window.  The tiled engine's
// M_SPARSE_SWA mode computes the same for fp32 and fp8 inputs.
//
// Design:
//  * A workgroup (4 waves) owns BQ queries x the G heads of one KV group,
//    row r = query r / G, head r % G, like the engine.  Each wave owns 32 rows
//    as two groups of 16 (the N of v_mfma_f32_16x16x32_bf16); a group skips
//    every tile that none of its queries selected, and window tiles that lie
//    outside all of its rows' windows.
//  * Key tiles (64 keys) go HBM -> LDS with global_load_lds_dwordx4: each lane
//    fetches any 16 bytes, the 64 lanes of one instruction fill 1 KiB of LDS in
//    lane order.  No staging registers and no VALU work; two LDS buffers, the
//    loads of tile n+1 in flight while tile n is computed, one barrier a tile.
//  * K and V sit in LDS row-major, [64 keys][D], with the 16-byte chunks of
//    each row XOR-swizzled so that the fragment reads below hit distinct
//    banks.  K fragments (A of S^T = K Q^T) are ds_read_b128.  V^T fragments
//    (A of O^T = V^T P^T) are read from row-major V with ds_read_b64_tr_b16:
//    within each 16-lane slice, lane i receives element i of the four 4-element
//    rows addressed by the slice, i.e. four consecutive keys of one d.
//  * P^T comes from the lane's own S^T accumulators: the PV k-dimension visits
//    the 64 keys in the order that matches the accumulator layout.
//  * The sparse branch's normalised output waits in registers (packed bf16)
//    while the window tiles run, so the output is written once (fp32 outputs
//    park it in the output row instead, as the engine does).
//
// v_mfma_f32_16x16x32_bf16 lane layout (wave64): lane l holds
// A[m = l%16][k = 8(l/16) + j], B[k = 8(l/16) + j][n = l%16] (j = 0..7) and
// C[m = 4(l/16) + i][n = l%16] (i = 0..3).
#include "common.h"
#include "kernels.h"
#include "block_union.h"
#include <type_traits>

namespace hys {
namespace {

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

template <int D> struct Geo {
  static constexpr int ROWB = 2 * D;            // bytes per key row
  static constexpr int CPR = D / 8;             // 16-byte chunks per row
  static constexpr int RPI = 1024 / ROWB;       // rows filled by one DMA instruction
  static constexpr int NU = 64 / (4 * RPI);     // DMA instructions per wave, operand and tile
  static constexpr int TILEB = 64 * ROWB;       // bytes of one operand tile
  static constexpr int NC = D / 32;             // k-steps of S^T
  static constexpr int NDB = D / 16;            // 16-wide d blocks of O^T
};

// chunk c of key row r is stored at chunk c ^ swz(r)
template <int D> __device__ __forceinline__ int swz_k(int r) { return r & (D / 8 - 1); }
template <int D> __device__ __forceinline__ int swz_v(int r) {
  return D == 128 ? 2 * (r & 3) + 8 * ((r >> 2) & 1) : 2 * (r & 3) + ((r >> 2) & 1);
}

__device__ __forceinline__ float xor16_sum(float v) { return v + __shfl_xor(v, 16); }
__device__ __forceinline__ float xor32_sum(float v) { return v + __shfl_xor(v, 32); }

// all LDS reads and writes of this wave, and this wave's LDS loads, are done;
// then the workgroup barrier (a compiler barrier for memory as well)
__device__ __forceinline__ void tile_barrier() {
  __builtin_amdgcn_s_waitcnt(0x0070);   // vmcnt(0) lgkmcnt(0)
  asm volatile("s_barrier" ::: "memory");
}

template <int D>
__global__ __launch_bounds__(256, 2) void sparse_layer_kernel(const AttnArgs a) {
  using P = Geo<D>;
  constexpr int UMAX = 512;      // union entries: BQ * topk <= 512 (host-checked)
  constexpr int NBWMAX = 512;    // bitmap words: nblk <= 16384 (host-checked)
  // two stages, each operand and stage its own array: every LDS access names
  // one of them statically (the tile loops are unrolled by two), which is what
  // lets the compiler tell the loads into one stage from the reads of the
  // other and keep the loads in flight across a whole tile
  __shared__ __attribute__((aligned(1024))) unsigned char K0[P::TILEB];
  __shared__ __attribute__((aligned(1024))) unsigned char K1[P::TILEB];
  __shared__ __attribute__((aligned(1024))) unsigned char V0[P::TILEB];
  __shared__ __attribute__((aligned(1024))) unsigned char V1[P::TILEB];
  __shared__ uint32_t s_bitmap[NBWMAX];
  __shared__ int s_wpre[NBWMAX];
  __shared__ int s_ulist[UMAX];
  __shared__ unsigned long long s_member[UMAX];
  __shared__ int s_count;

  const int tid = threadIdx.x, lane = tid & 63;
  // the wave index as a scalar, so that every per-wave quantity below is too
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int li = lane & 15, lg = lane >> 4;
  if ((int)blockIdx.x >= a.grid_used) return;

  // ---- work item: KV group fastest, longest query tiles first ---------------
  const int g = (int)blockIdx.x % a.Hkv;
  const int rest = (int)blockIdx.x / a.Hkv;
  const int b = rest % a.B;
  const int qt = a.ntq - 1 - rest / a.B;
  const int q0 = qt * a.BQ;
  const int nq = min(a.BQ, a.Lq - q0);          // queries of this workgroup
  const int qa0 = q0 + a.q_off, qa_last = q0 + nq - 1 + a.q_off;
  const int HC = a.HC;

  // ---- rows: group gi of this wave is rows wave*32 + gi*16 + (0..15); the
  // lane's row is li, its slice lg holds d values of that row ----------------
  int qpos[2], head[2], qiv[2];
  bool valid[2], gany[2];
  unsigned long long gmask[2];
  int glo[2], ghi[2];
#pragma unroll
  for (int gi = 0; gi < 2; ++gi) {
    const int r0 = wave * 32 + gi * 16;
    const int r = r0 + li;
    const int qi = r / HC;
    qiv[gi] = qi;
    qpos[gi] = q0 + qi;
    head[gi] = g * a.G + (r - qi * HC);
    valid[gi] = qi < nq;
    const int qlo = r0 / HC, qhi = min((r0 + 15) / HC, nq - 1);
    gany[gi] = qlo <= qhi;
    gmask[gi] = gany[gi] ? (((qhi - qlo == 63) ? ~0ull : ((1ull << (qhi - qlo + 1)) - 1ull)) << qlo) : 0ull;
    glo[gi] = q0 + qlo + a.q_off - a.window + 1;   // window keys seen by some row of the group
    ghi[gi] = q0 + qhi + a.q_off;
  }

  // ---- Q fragments (B of S^T): q[row][32c + 8lg .. +7] ----------------------
  const uint16_t* qbase = (const uint16_t*)a.q + (int64_t)b * a.q_sb;
  bf16x8 qf[2][P::NC];
#pragma unroll
  for (int gi = 0; gi < 2; ++gi) {
    const uint16_t* qr = qbase + (valid[gi] ? (int64_t)qpos[gi] * a.q_st + (int64_t)head[gi] * a.q_sh : 0);
#pragma unroll
    for (int c = 0; c < P::NC; ++c) {
      const uint4 x = *(const uint4*)(qr + 32 * c + 8 * lg);
      const uint4 z = {0u, 0u, 0u, 0u};
      qf[gi][c] = as_bf16x8(valid[gi] ? x : z);
    }
  }

  // ---- the workgroup's selected blocks, then its window tiles ---------------
  const int32_t* ib = a.idx + (int64_t)b * a.idx_sb + (int64_t)g * a.idx_sg;
  const int nsp = __builtin_amdgcn_readfirstlane(build_block_union<UMAX, NBWMAX>(
      ib, a.idx_sr, a.topk, q0, a.BQ, a.Lq, a.nblk, s_bitmap, s_wpre, s_ulist, s_member, &s_count));
  const int wstart = max(0, qa0 - a.window + 1);
  const int wend = min(qa_last, a.Lk - 1);
  const int ntiles = nsp + (wend - wstart + 1 + 63) / 64;

  // ---- tile loads ---------------------------------------------------------
  const uint16_t* kb = (const uint16_t*)a.k + (int64_t)b * a.k_sb + (int64_t)g * a.k_sh;
  const uint16_t* vb = (const uint16_t*)a.v + (int64_t)b * a.v_sb + (int64_t)g * a.v_sh;
  const uint16_t* kwb = (const uint16_t*)a.kw + (int64_t)b * a.k_sb + (int64_t)g * a.k_sh;
  const uint16_t* vwb = (const uint16_t*)a.vw + (int64_t)b * a.v_sb + (int64_t)g * a.v_sh;
  // instruction u of this wave fills tile rows (4u + wave) * RPI + (0..RPI-1);
  // a swizzle depends on the row mod 16, and 4 * RPI is a multiple of 16, so
  // the chunk a lane fetches is the same for every u.  The lane's byte offset
  // from a tile's first key row is fixed; the rest of an address is scalar.
  // (64 rows of K or V span less than 2^32 bytes: checked by the host.)
  const int drow0 = wave * P::RPI + lane / P::CPR;
  const uint32_t kstb = (uint32_t)a.k_st * 2u, vstb = (uint32_t)a.v_st * 2u;
  const uint32_t chunk_k = (uint32_t)(((lane % P::CPR) ^ swz_k<D>(drow0)) * 16);
  const uint32_t chunk_v = (uint32_t)(((lane % P::CPR) ^ swz_v<D>(drow0)) * 16);
  const uint32_t lane_k = (uint32_t)drow0 * kstb + chunk_k;
  const uint32_t lane_v = (uint32_t)drow0 * vstb + chunk_v;
  // first key of tile n (scalar)
  auto tile_first = [&](int n) __attribute__((always_inline)) -> int {
    return n >= nsp ? wstart + (n - nsp) * 64 : __builtin_amdgcn_readfirstlane(s_ulist[n]) * 64;
  };
  auto load_tile = [&](int n, int j0, unsigned char* Kd, unsigned char* Vd) __attribute__((always_inline)) {
    const bool own = n >= nsp;
    const int jlast = own ? wend : a.Lk - 1;
    const char* kt = (const char*)(own ? kwb : kb) + (int64_t)j0 * a.k_st * 2;
    const char* vt = (const char*)(own ? vwb : vb) + (int64_t)j0 * a.v_st * 2;
    if (j0 + 63 <= jlast) {
      // whole tile: a scalar base per instruction + the lane's fixed offset
      // (the saddr form; the two offset registers stay live through the loops)
#pragma unroll
      for (int u = 0; u < P::NU; ++u) {
        const char* ktu = kt + (int64_t)(4 * P::RPI * u) * a.k_st * 2;
        const char* vtu = vt + (int64_t)(4 * P::RPI * u) * a.v_st * 2;
        __builtin_amdgcn_global_load_lds((const void*)(ktu + lane_k), (lds_void*)(Kd + (4 * u + wave) * 1024), 16, 0, 0);
        __builtin_amdgcn_global_load_lds((const void*)(vtu + lane_v), (lds_void*)(Vd + (4 * u + wave) * 1024), 16, 0, 0);
      }
    } else {
      // partial tile: slots past the last key repeat the last key's row
      // (their logits are masked, so their probabilities are exactly 0)
      const int rmax = jlast - j0;
#pragma unroll
      for (int u = 0; u < P::NU; ++u) {
        const uint32_t rr = (uint32_t)min(drow0 + 4 * P::RPI * u, rmax);
        __builtin_amdgcn_global_load_lds((const void*)(kt + (rr * kstb + chunk_k)), (lds_void*)(Kd + (4 * u + wave) * 1024), 16, 0, 0);
        __builtin_amdgcn_global_load_lds((const void*)(vt + (rr * vstb + chunk_v)), (lds_void*)(Vd + (4 * u + wave) * 1024), 16, 0, 0);
      }
    }
  };

  // per-lane LDS byte offsets of the fragments inside a tile.  The swizzles
  // only flip the bits that select the k-step (K: 64-byte units) or the d block
  // (V: 32-byte units) within the lane's offset, so the offset of step c / block
  // db is the lane's base XOR 64c / 32db.
  //   K, row 16kb + li, chunk 4c + lg:  li*ROWB + 16*((4c + lg) ^ swz_k(li))
  //   V, rows 16(2ks+h) + kr, d 16db + 4(li%4) .. +3 with kr = 4lg + li/4:
  //      kr*ROWB + 16*((2db + (li/2)%2) ^ swz_v(kr)) + 8*(li%2)
  const int kbase_off = li * P::ROWB + (((lg) ^ swz_k<D>(li)) * 16);
  int vbase_off;
  {
    const int kr = 4 * lg + (li >> 2);
    vbase_off = kr * P::ROWB + ((((li >> 1) & 1) ^ swz_v<D>(kr)) * 16) + (li & 1) * 8;
  }
  // ---- softmax state -------------------------------------------------------
  const float c2 = a.scale_log2;
  const float lazy_raw = kLazyLog2 / c2;
  float m_run[2], l_run[2];
  f32x4 acc[2][P::NDB];
  uint32_t osp[2][P::NDB][2];     // sparse branch, packed bf16 (bf16 outputs)
  bool sp_live[2];
#pragma unroll
  for (int gi = 0; gi < 2; ++gi) {
    m_run[gi] = kNegInf; l_run[gi] = 0.f; sp_live[gi] = false;
#pragma unroll
    for (int db = 0; db < P::NDB; ++db) {
      acc[gi][db] = f32x4{0.f, 0.f, 0.f, 0.f};
      osp[gi][db][0] = osp[gi][db][1] = 0u;
    }
  }
  auto row_off = [&](int gi) __attribute__((always_inline)) -> int64_t {
    return (int64_t)b * a.o_sb + (int64_t)qpos[gi] * a.o_st + (int64_t)head[gi] * a.o_sh;
  };
  // end of the selected blocks: normalise and park the sparse branch, restart
  // the softmax state for the window
  auto finish_sparse = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int gi = 0; gi < 2; ++gi) {
      const float lsum = xor32_sum(xor16_sum(l_run[gi]));
      sp_live[gi] = m_run[gi] != kNegInf;
      const float inv = sp_live[gi] ? a.v_scale / lsum : 0.f;
#pragma unroll
      for (int db = 0; db < P::NDB; ++db) {
        const f32x4 r = acc[gi][db] * inv;
        if (a.o_f32) {
          if (valid[gi]) *(f32x4*)((float*)a.o + row_off(gi) + 16 * db + 4 * lg) = r;
        } else {
          osp[gi][db][0] = pack_bf16x2(r[0], r[1]);
          osp[gi][db][1] = pack_bf16x2(r[2], r[3]);
        }
        acc[gi][db] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
      m_run[gi] = kNegInf; l_run[gi] = 0.f;
    }
  };

  // ---- one tile ---------------------------------------------------------------
  // Kc/Vc: the tile being computed; Kn/Vn: the buffer the next tile is loaded
  // into.  They never overlap; passing them as restrict arguments tells the
  // compiler so, and it then lets the loads stay in flight across this tile's
  // LDS reads (the barrier at the end waits for them explicitly).
  // OWN: a window tile of the layer's own K/V (else a selected block)
  auto step = [&](auto own_tag, int n, const unsigned char* __restrict__ Kc, const unsigned char* __restrict__ Vc,
                  unsigned char* __restrict__ Kn, unsigned char* __restrict__ Vn) __attribute__((always_inline)) {
    constexpr bool own = decltype(own_tag)::value;
    // the fragment offsets of the tile are XORs of these bases; recomputing
    // them each tile keeps them out of the loops' register budget
    int kbo = kbase_off, vbo = vbase_off;
    asm volatile("" : "+v"(kbo), "+v"(vbo));
    const int j0 = tile_first(n);
    unsigned long long memb = 0ull;
    if (!own) {
      const unsigned long long m = s_member[n];
      memb = ((unsigned long long)__builtin_amdgcn_readfirstlane((uint32_t)(m >> 32)) << 32) |
             (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)m);
    }
    const int j0n = n + 1 < ntiles ? tile_first(n + 1) : 0;
    // the list reads above stay ahead of the loads below (no load is pending
    // here, so they need no wait)
    asm volatile("" ::: "memory");
    if (n + 1 < ntiles) load_tile(n + 1, j0n, Kn, Vn);

    bool act[2], row_on[2], emask[2];
    int lo[2], hi[2];
#pragma unroll
    for (int gi = 0; gi < 2; ++gi) {
      act[gi] = gany[gi] && (own ? (j0 <= ghi[gi] && j0 + 63 >= glo[gi]) : ((memb & gmask[gi]) != 0ull));
      row_on[gi] = valid[gi] && (own || ((memb >> qiv[gi]) & 1ull) != 0ull);
      hi[gi] = qpos[gi] + a.q_off;
      lo[gi] = own ? hi[gi] - a.window + 1 : 0;
      const bool part = row_on[gi] && !(j0 >= lo[gi] && j0 + 63 <= hi[gi]);
      emask[gi] = __ballot(part) != 0ull;
    }

    // One code path for every combination of active groups: each group's MFMAs
    // and softmax sit behind a scalar branch on act[gi], so its registers are
    // updated in place or left alone (separate code paths per combination made
    // the compiler copy the accumulators at every join).
    auto body = [&]() __attribute__((always_inline)) {
      const bool* ACT = act;
      // S^T = K Q^T: 4 key blocks of 16 x NC k-steps of 32 d; the K fragments
      // (shared by both groups) of step c+1 are read while step c's MFMAs issue
      f32x4 s[2][4];
      uint4 kf[2][4];
      auto kload = [&](int c, uint4(&dst)[4]) __attribute__((always_inline)) {
#pragma unroll
        for (int kb4 = 0; kb4 < 4; ++kb4) dst[kb4] = *(const uint4*)(Kc + (kbo ^ (64 * c)) + kb4 * 16 * P::ROWB);
      };
      kload(0, kf[0]);
#pragma unroll
      for (int c = 0; c < P::NC; ++c) {
        if (c + 1 < P::NC) kload(c + 1, kf[(c + 1) & 1]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int gi = 0; gi < 2; ++gi)
          if (ACT[gi]) {
#pragma unroll
            for (int kb4 = 0; kb4 < 4; ++kb4)
              s[gi][kb4] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kf[c & 1][kb4]), qf[gi][c],
                                                                   c == 0 ? f32x4{0.f, 0.f, 0.f, 0.f} : s[gi][kb4],
                                                                   0, 0, 0);
          }
      }
      // V^T fragments of d block db: ks-th k-step from two transposing reads
      bf16x8 vf[2][2];
      auto vload = [&](int db, bf16x8(&dst)[2]) __attribute__((always_inline)) {
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const v4i16 t0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_v4i16*)(Vc + (vbo ^ (32 * db)) + (32 * ks) * P::ROWB));
          const v4i16 t1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_v4i16*)(Vc + (vbo ^ (32 * db)) + (32 * ks + 16) * P::ROWB));
          const uint2 u0 = __builtin_bit_cast(uint2, t0), u1 = __builtin_bit_cast(uint2, t1);
          dst[ks] = as_bf16x8(make_uint4(u0.x, u0.y, u1.x, u1.y));
        }
      };
      // the first d block's reads hide under the softmax
      vload(0, vf[0]);
      __builtin_amdgcn_sched_barrier(0);

      // online softmax (base 2 on raw dot products, lazily moved reference);
      // lane (li, lg) holds keys 16kb + 4lg + i of row li
      bf16x8 pf[2][2];
#pragma unroll
      for (int gi = 0; gi < 2; ++gi) {
        if (!ACT[gi]) continue;
        if (emask[gi]) {
          const unsigned span = (unsigned)(hi[gi] - lo[gi]);
#pragma unroll
          for (int kb4 = 0; kb4 < 4; ++kb4)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int key = j0 + 16 * kb4 + 4 * lg + i;
              const bool ok = row_on[gi] & ((unsigned)(key - lo[gi]) <= span);
              s[gi][kb4][i] = ok ? s[gi][kb4][i] : kNegInf;
            }
        }
        // row maximum: three-input maxima (no NaN quieting of the MFMA results)
        float mk[4];
#pragma unroll
        for (int kb4 = 0; kb4 < 4; ++kb4)
          mk[kb4] = fmax_nc(fmax_nc(s[gi][kb4][0], s[gi][kb4][1]), fmax_nc(s[gi][kb4][2], s[gi][kb4][3]));
        float mt = fmax_nc(fmax_nc(mk[0], mk[1]), fmax_nc(mk[2], mk[3]));
        mt = xor32_max(xor16_max(mt));
        if (!row_on[gi]) mt = kNegInf;
        // the reference moves (and O, l are rescaled) only in the rare tiles
        // where some row's maximum exceeds it by more than the slack
        const bool need = mt > m_run[gi] + lazy_raw;
        float alpha = 1.f;
        if (__ballot(need) != 0ull) {
          const float mref = need ? mt : m_run[gi];
          alpha = need ? __builtin_amdgcn_exp2f((m_run[gi] - mref) * c2) : 1.f;
          m_run[gi] = mref;
#pragma unroll
          for (int db = 0; db < P::NDB; ++db) acc[gi][db] *= alpha;
        }
        const float mref = m_run[gi];
        const float mc = !row_on[gi] ? __builtin_huge_valf() : ((mref == kNegInf) ? 0.f : mref * c2);
        float pk4[4];
#pragma unroll
        for (int kb4 = 0; kb4 < 4; ++kb4) {
#pragma unroll
          for (int i = 0; i < 4; ++i) s[gi][kb4][i] = __builtin_amdgcn_exp2f(fmaf(s[gi][kb4][i], c2, -mc));
          pk4[kb4] = (s[gi][kb4][0] + s[gi][kb4][1]) + (s[gi][kb4][2] + s[gi][kb4][3]);
        }
        const float ps = (pk4[0] + pk4[1]) + (pk4[2] + pk4[3]);
        l_run[gi] = fmaf(l_run[gi], alpha, ps);
        // PV k-step ks: k = 8lg + j <-> key 16(2ks + j/4) + 4lg + j%4
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          uint4 pk;
          pk.x = pack_bf16x2(s[gi][2 * ks][0], s[gi][2 * ks][1]);
          pk.y = pack_bf16x2(s[gi][2 * ks][2], s[gi][2 * ks][3]);
          pk.z = pack_bf16x2(s[gi][2 * ks + 1][0], s[gi][2 * ks + 1][1]);
          pk.w = pack_bf16x2(s[gi][2 * ks + 1][2], s[gi][2 * ks + 1][3]);
          pf[gi][ks] = as_bf16x8(pk);
        }
      }

      // O^T += V^T P^T, one 16-wide d block at a time, the next block's V^T read ahead
#pragma unroll
      for (int db = 0; db < P::NDB; ++db) {
        if (db + 1 < P::NDB) vload(db + 1, vf[(db + 1) & 1]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int gi = 0; gi < 2; ++gi)
          if (ACT[gi]) {
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
              acc[gi][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf[db & 1][ks], pf[gi][ks], acc[gi][db], 0, 0, 0);
          }
      }
    };
    if (act[0] || act[1]) body();
    tile_barrier();
  };

  // ---- tile loop ---------------------------------------------------------------
  // (two loops, so that the switch between the branches is not a branch inside one)
  load_tile(0, tile_first(0), K0, V0);
  tile_barrier();
  // tile n is computed from stage n & 1
  int n = 0;
  for (; n + 1 < nsp; n += 2) {
    step(std::false_type{}, n, K0, V0, K1, V1);
    step(std::false_type{}, n + 1, K1, V1, K0, V0);
  }
  if (n < nsp) {
    step(std::false_type{}, n, K0, V0, K1, V1);
    ++n;
  }
  finish_sparse();
  if ((n & 1) && n < ntiles) {
    step(std::true_type{}, n, K1, V1, K0, V0);
    ++n;
  }
  for (; n < ntiles; n += 2) {
    step(std::true_type{}, n, K0, V0, K1, V1);
    if (n + 1 < ntiles) step(std::true_type{}, n + 1, K1, V1, K0, V0);
  }

  // ---- epilogue: window branch, gate, one store per row ----------------------
#pragma unroll
  for (int gi = 0; gi < 2; ++gi) {
    const float lsum = xor32_sum(xor16_sum(l_run[gi]));
    const bool live = m_run[gi] != kNegInf;
    const float inv = live ? a.v_scale / lsum : 0.f;
    // g = sigmoid(<q, w_h> + b_h) over d = 32c + 8lg + (0..7) of the lane's row
    // (q is read again rather than kept live across the tile loop)
    float z = 0.f;
    if (valid[gi]) {
      const float* w = a.gate_w + (int64_t)head[gi] * D;
      const uint16_t* qr = qbase + (int64_t)qpos[gi] * a.q_st + (int64_t)head[gi] * a.q_sh;
#pragma unroll
      for (int c = 0; c < P::NC; ++c) {
        const uint4 qv = *(const uint4*)(qr + 32 * c + 8 * lg);
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const uint32_t wv = u4get(qv, p);
          z = fmaf(bf16_to_f32((uint16_t)(wv & 0xffffu)), w[32 * c + 8 * lg + 2 * p], z);
          z = fmaf(bf16_to_f32((uint16_t)(wv >> 16)), w[32 * c + 8 * lg + 2 * p + 1], z);
        }
      }
    }
    z = xor32_sum(xor16_sum(z));
    if (!valid[gi]) continue;
    if (a.gate_b) z += a.gate_b[head[gi]];
    const float gate = 1.f / (1.f + __expf(-z));
    const int64_t ro = row_off(gi);
#pragma unroll
    for (int db = 0; db < P::NDB; ++db) {
      const int d = 16 * db + 4 * lg;
      f32x4 r = acc[gi][db] * inv;
      if (sp_live[gi]) {
        f32x4 sp;
        if (a.o_f32) {
          sp = *(const f32x4*)((const float*)a.o + ro + d);
        } else {
          sp[0] = bf16_to_f32((uint16_t)(osp[gi][db][0] & 0xffffu));
          sp[1] = bf16_to_f32((uint16_t)(osp[gi][db][0] >> 16));
          sp[2] = bf16_to_f32((uint16_t)(osp[gi][db][1] & 0xffffu));
          sp[3] = bf16_to_f32((uint16_t)(osp[gi][db][1] >> 16));
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) r[e] = gate * sp[e] + (1.f - gate) * r[e];
      }
      if (a.o_f32) {
        *(f32x4*)((float*)a.o + ro + d) = r;
      } else {
        uint2 out;
        out.x = pack_bf16x2(r[0], r[1]);
        out.y = pack_bf16x2(r[2], r[3]);
        *(uint2*)((uint16_t*)a.o + ro + d) = out;
      }
    }
  }
}

}  // namespace

hipError_t launch_sparse_layer(int D, const AttnArgs& a, int grid, hipStream_t s) {
  if (a.HC != a.G || a.BQ < 1 || a.BQ > 64 || a.BQ * a.topk > 512 || a.nblk > 16384)
    return hipErrorInvalidValue;
  if (D == 64) hipLaunchKernelGGL(sparse_layer_kernel<64>, dim3(grid), dim3(256), 0, s, a);
  else if (D == 128) hipLaunchKernelGGL(sparse_layer_kernel<128>, dim3(grid), dim3(256), 0, s, a);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace hys
