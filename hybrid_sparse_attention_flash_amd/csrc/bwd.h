// Internal launch interface of the backward-pass kernels (gfx950).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hys {

// Which keys a query row sees in one attention branch.
enum BwdMode {
  BW_CAUSAL = 0,   // j <= i (the full layer)
  BW_WINDOW = 1,   // i - window < j <= i (the window branch over the layer's own K/V)
  BW_BLOCK = 2,    // j <= i and block j/64 selected by row i (the block-sparse branch)
};

struct BwdArgs {
  const uint16_t* q; int64_t q_sb, q_st, q_sh;      // [B, L, Hq, D] bf16
  const uint16_t* k; const uint16_t* v;             // [B, Lk, Hkv, D] bf16, one set of strides
  int64_t k_sb, k_st, k_sh;
  const uint16_t* dO; int64_t do_sb, do_st, do_sh;  // upstream gradient of this branch, bf16
  const float* lse;                                 // [B, Hq, L] natural-log LSE of this branch
  const float* Dd;                                  // [B, Hq, L] rowsum(dO * O) of this branch
  float* dq; int64_t dq_sb, dq_st, dq_sh;           // fp32
  float* dk; float* dv; int64_t dk_sb, dk_st, dk_sh;   // fp32, one set of strides
  int B, L, Lk, Hq, Hkv, G;
  float scale, scale_log2;
  int window;
  // BW_BLOCK: selection bitmaps (bit c of word c/32 = block c selected)
  const uint32_t* rowbits;    // [ng][B][nwords][L]: per query row (word-major)
  // the query rows (ascending, rows >= the block's first key) that selected
  // 64-key block c: rowlist [ng][B][nblk][L], rowcnt [ng][B][nblk] entries
  // used, nblk = ceil(Lk/64)
  const int32_t* rowlist; const int32_t* rowcnt;
  const uint32_t* tilebits16; // [ng][B][ceil(L/16)][nwords]: OR over the 16-row blocks
  int nwords, ng;             // ng = 1 (one set for every KV group) or Hkv
  int acc_q, acc_kv;          // 1: add into dq / dk, dv; 0: overwrite
  // dK/dV row split: the query rows a 64-key block sees (block mode: its row
  // list) are cut into nsplit ranges of split_rb * 32 rows counted from the
  // block's first, one workgroup each; with nsplit > 1 each writes
  // its partial sums (part_k, part_v: [nsplit][B][Lk][Hkv][D] fp32) and a flag
  // (flags: one per workgroup), and a reduce pass adds the flagged partials
  // into dk, dv in split order
  int nsplit, split_rb;
  float* part_k; float* part_v; int32_t* flags;
};

// Row split of the dK/dV pass for a branch: returns nsplit (1 = no split) and
// the row blocks per split, and the workspace bytes it needs.
int bwd_dkdv_plan(int mode, int L, int window, int* split_rb);
size_t bwd_dkdv_ws_bytes(int nsplit, int B, int Lk, int Hkv, int D);
// points part_k, part_v, flags into ws (bwd_dkdv_ws_bytes bytes, 16-byte aligned)
void bwd_dkdv_bind_ws(BwdArgs& a, void* ws, int D);

hipError_t launch_bwd_dkdv(int mode, int D, const BwdArgs& a, hipStream_t s);
hipError_t launch_bwd_dq(int mode, int D, const BwdArgs& a, hipStream_t s);

// rowsum(dO * O) per (b, h, i) for the full layer: [B, Hq, L]
struct BwdPrepArgs {
  const void* dO; int64_t do_sb, do_st, do_sh; int do_f32;
  const void* o; int64_t o_sb, o_st, o_sh; int o_f32;
  float* Dd;
  int B, L, Hq, D;
};
hipError_t launch_bwd_prep_full(const BwdPrepArgs& a, hipStream_t s);

// Sparse-layer gate: per (b, i, h) g = sigmoid(<q, w_h> + b_h), the branch
// gradients dO_sp = g dO and dO_w = (1 - g) dO (bf16, contiguous [B, L, Hq, D]),
// their rowsums with the branch outputs, dz = g (1 - g) <dO, O_sp - O_w>, and
// dq = dz w_h (written).  A row without a sparse branch (lse_sp = -inf) takes g = 0.
struct BwdGateArgs {
  const uint16_t* q; int64_t q_sb, q_st, q_sh;
  const void* dO; int64_t do_sb, do_st, do_sh; int do_f32;
  const void* osp; int64_t osp_sb, osp_st, osp_sh; int osp_f32;
  const void* ow; int64_t ow_sb, ow_st, ow_sh; int ow_f32;
  const float* lse_sp;                          // [B, Hq, L]
  const float* gate_w; const float* gate_b;     // [Hq, D], [Hq] or null
  uint16_t* do_sp; uint16_t* do_w;              // [B, L, Hq, D] bf16
  float* Dd_sp; float* Dd_w; float* dz;         // [B, Hq, L]
  float* dq; int64_t dq_sb, dq_st, dq_sh;
  int B, L, Hq, D;
};
hipError_t launch_bwd_prep_gate(const BwdGateArgs& a, hipStream_t s);

// dgate_w[h][d] = sum over (b, i) of dz[b, h, i] * q[b, i, h, d] and, when
// dgate_b is not null, dgate_b[h] = sum over (b, i) of dz[b, h, i], in fixed
// order: partial sums over row splits into `part` (bwd_gate_partial_floats
// floats), then their sum
size_t bwd_gate_partial_floats(int Hq, int D);
hipError_t launch_bwd_gate_grad(const float* dz, const uint16_t* q, int64_t q_sb, int64_t q_st, int64_t q_sh,
                                int B, int L, int Hq, int D, float* part, float* dgate_w, float* dgate_b,
                                hipStream_t s);

// selection bitmaps from block ids idx[g*idx_sg + b*idx_sb + i*idx_sr + j] (j < k; -1 = unused),
// then the per-block row lists of the dK/dV pass (nblk blocks of 64 keys)
hipError_t launch_bwd_selbits(const int32_t* idx, int64_t idx_sg, int64_t idx_sb, int64_t idx_sr, int k, int ng,
                              int B, int L, int nblk, int nwords, uint32_t* rowbits, uint32_t* tilebits16,
                              int32_t* rowlist, int32_t* rowcnt, hipStream_t s);

}  // namespace hys
