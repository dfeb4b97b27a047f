// Internal launch interface between the C-ABI layer and the gfx950 kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hys {

enum ElemType { ET_F32 = 0, ET_BF16 = 1, ET_FP8 = 2 };

// Prefill attention modes, all served by one tiled MFMA engine.
enum AttnMode {
  M_FULL = 0,          // causal attention, no scores
  M_FULL_BLOCK = 1,    // causal attention + per-(query, key-block) max logit
  M_FULL_TILE = 2,     // causal attention + per-(query-tile, key) max logit
  M_SPARSE_BLOCK = 3,  // attention over selected key blocks (per-query selection)
  M_SPARSE_TOKEN = 4,  // attention over selected tokens of a query tile + forced recent window
  M_SWA_GATE = 5,      // sliding-window attention fused with the sigmoid gate merge
  M_SPARSE_SWA = 6,    // selected key blocks, then the layer's own window, merged by the gate
};

struct AttnArgs {
  const void* q; int64_t q_sb, q_st, q_sh;
  const void* k; int64_t k_sb, k_st, k_sh;
  const void* v; int64_t v_sb, v_st, v_sh;
  void* o; int64_t o_sb, o_st, o_sh;
  int o_f32;                 // 1: fp32 output, 0: bf16 output
  float* lse;                // [B, Hq, Lq] or null
  int B, Lq, Lk, Hq, Hkv, G;
  int q_off;                 // absolute position of query row 0 (chunked prefill); masks use q_off + row
  float scale_log2;          // softmax scale * k scale * log2(e)
  float logit_scale;         // softmax scale * k scale
  float v_scale;             // V dequantisation scale applied to O
  int BQ;                    // queries per workgroup row set
  int HC;                    // query heads per row set
  int nhc;                   // head chunks per KV group = ceil(G / HC)
  int ntq;                   // number of query tiles = ceil(Lq / BQ)
  // importance scores (M_FULL_BLOCK: [B, Lq, nblk] per KV group slab; M_FULL_TILE: [B, ntq, Lk])
  float* scores; int64_t sc_sb, sc_sr, sc_sg;
  int nblk;
  // sparse selection
  const int32_t* idx; int64_t idx_sb, idx_sr;
  int64_t idx_sg;            // between KV groups' index rows (0: one selection for every group)
  int topk;
  int window;
  // the layer's own window K/V (M_SPARSE_SWA; same strides as k, v)
  const void* kw; const void* vw;
  // gate inputs (M_SWA_GATE, M_SPARSE_SWA)
  const float* o_sp; int64_t osp_sb, osp_st, osp_sh;
  const float* lse_sp;       // [B, Hq, Lq]
  const float* gate_w;       // [Hq, D]
  const float* gate_b;       // [Hq] or null
  int grid_used;             // work items; extra workgroups exit
  int nb;                    // 32-row MFMA blocks per wave: 1 (128 rows per workgroup)
};

hipError_t launch_attn(int mode, int qt, int kt, int D, const AttnArgs& a, int grid, hipStream_t s);

// The one-pass sparse layer (M_SPARSE_SWA's computation) for bf16 q/k/v, fp32
// or bf16 output; needs HC == G, BQ * topk <= 512, nblk <= 16384, D 64 or 128.
hipError_t launch_sparse_layer(int D, const AttnArgs& a, int grid, hipStream_t s);

// The full layer (M_FULL, or M_FULL_BLOCK with scores) for bf16 q/k/v, fp32
// or bf16 output: D 64 or 128, HC == G, BQ == kFullLayerRows / G, and with
// scores 32 % G == 0.
constexpr int kFullLayerRows = 256;
bool full_layer_supported(int D, const AttnArgs& a, bool scores);
hipError_t launch_full_layer(int D, const AttnArgs& a, bool scores, int grid, hipStream_t s);

// M_FULL_TILE score rows [B, ntq, Lk] (row stride sr, batch stride sb):
// decode = 0 clears them to atomic-max keys, decode = 1 turns keys into fp32
hipError_t launch_tile_scores(float* sc, int B, int ntq, int BQ, int Lq, int Lk, int q_off, int64_t sb, int64_t sr,
                              int decode, hipStream_t s);

hipError_t launch_reduce_max(const float* part, int nparts, int64_t part_stride, float* out, int64_t n,
                             hipStream_t s);

struct TopkArgs {
  const float* scores; int64_t rows, cols, row_stride;
  int k;
  int32_t* idx; int32_t* count;
  // long rows (cols > topk_chunk_cols()): topk_workspace_bytes of 4-byte
  // aligned workspace for the row histograms, selection state and chunk counts;
  // hist_zeroed: its first topk_zero_ints ints are already 0 (else cleared here)
  void* ws;
  bool hist_zeroed;
};
hipError_t launch_topk(const TopkArgs& a, hipStream_t s);
// workspace of launch_topk for [rows, cols] and k; 0 when cols <= topk_chunk_cols()
size_t topk_workspace_bytes(int64_t rows, int64_t cols, int k);
// ints at the start of that workspace that must be 0 when the selection starts
int64_t topk_zero_ints(int64_t rows, int64_t cols);
// largest grid (workgroups) launch_topk uses
int64_t topk_max_workgroups(int64_t rows, int64_t cols, int k);
int64_t topk_chunk_cols();
hipError_t launch_fill_i32(int32_t* p, int32_t v, int64_t n, hipStream_t s);

// block-level selection over token-score rows: block maxima, then the chosen
// blocks expanded to token positions
hipError_t launch_block_max_rows(const float* scores, int64_t rows, int64_t cols, int64_t row_stride, int nblk,
                                 float* out, hipStream_t s);
hipError_t launch_expand_blocks(const int32_t* blocks, int64_t rows, int kb, int64_t cols, int32_t* idx,
                                hipStream_t s);

// HySparse2 decode (one query per sequence, MQA cache).
constexpr int kMaxDecodeLayers = 16;
constexpr int kMaxDecodeBatch = 64;

struct DecArgs {
  const void* q[kMaxDecodeLayers]; int64_t q_sb, q_sh;   // per layer [B, 1, Hq, D] bf16
  const void* k; int64_t k_sb, k_st;                     // [B, Nmax, 1, D]
  const void* v; int64_t v_sb, v_st;
  int lens[kMaxDecodeBatch];                             // valid cache length per sequence
  int B, Hq, Nmax, nsplit, nlayer;
  int ncu;                                               // compute units of the device
  float scale_log2, logit_scale;
  float* scores; int64_t sc_sb;                          // full mode: [B, Nmax] token scores
  const int32_t* idx; int64_t idx_sb; int topk; int window;   // sparse mode: [B, topk]
  float* part_o; float* part_ml;                         // [(layer*B + b)*nsplit + s][Hq][D], [..][Hq][2]
  int32_t* zero; int64_t zero_n;                         // full mode: ints cleared for a later launch (or null)
  // full mode with nlayer > 1 (one "layer" per KV head of a GQA cache): element
  // offsets of layer l's K, V and score rows (0 for a single layer)
  int64_t k_sl, v_sl, sc_sl;
};

struct MergeArgs {
  const float* part_o; const float* part_ml;
  int B, Hq, nsplit, nlayer;
  float logit_scale, v_scale, scale_log2;
  void* o[kMaxDecodeLayers]; int64_t o_sb, o_sh; int o_f32;
  float* lse[kMaxDecodeLayers];                          // [B, Hq] per layer or null
};

hipError_t launch_decode(int sparse, int kt, int D, const DecArgs& a, hipStream_t s);
hipError_t launch_decode_merge(int D, const MergeArgs& a, hipStream_t s);
// two merges in one launch: the workgroups of a, then those of b
hipError_t launch_decode_merge2(int D, const MergeArgs& a, const MergeArgs& b, hipStream_t s);

// HySparse (block-level) decode: block scores from the full layer's per-KV-head
// token scores, and every sparse layer (block gather, ring window, gate).
hipError_t launch_hs_block_max(const float* ts, int nparts, int64_t part_stride, int B, int Nmax, int nblk,
                               float* out, hipStream_t s);

struct HsDecArgs {
  const uint16_t* k; int64_t k_sb, k_st, k_sh;           // shared cache [B, Nmax, Hkv, D] bf16
  const uint16_t* v; int64_t v_sb, v_st, v_sh;
  int lens[kMaxDecodeBatch];
  int B, Hkv, G, nlayer, topk, W;                        // G query heads per KV head, W ring slots
  float scale_log2;                                      // softmax scale * log2(e)
  const int32_t* idx; int64_t idx_sb;                    // [B, topk] selected block ids
  const uint16_t* q[kMaxDecodeLayers]; int64_t q_sb, q_sh;        // [B, 1, Hq, D] bf16 per layer
  const uint16_t* knew[kMaxDecodeLayers]; const uint16_t* vnew[kMaxDecodeLayers];
  int64_t n_sb, n_sh;                                    // new token's window K/V [B, 1, Hkv, D]
  uint16_t* kring[kMaxDecodeLayers]; uint16_t* vring[kMaxDecodeLayers];
  int64_t r_sb, r_st, r_sh;                              // rings [B, W, Hkv, D]
  const float* gate_w[kMaxDecodeLayers];                 // [Hq, D] fp32 per layer
  void* o[kMaxDecodeLayers]; int64_t o_sb, o_sh; int o_f32;       // [B, 1, Hq, D]
  // split over workgroups: splits 0..nsplit-2 take 4 selected blocks each, the
  // last the window; part [nlayer][B][Hq][nsplit][2 + D]: base-2 max M, sum L,
  // normalised O of each split, merged with the gate by a second kernel
  int nsplit; float* part;
};
int hs_decode_splits(int topk);
hipError_t launch_hs_decode_sparse(int D, const HsDecArgs& a, hipStream_t s);

// HySparse2 KV Bridging: K/V of a cross-decoder full layer projected from
// hidden states straight into the fp8 e4m3 cache.
struct BridgeArgs {
  const void* h; int64_t h_sb, h_st;                    // [B, L, 1, d_model] bf16
  const void* w_k; const void* w_v;                     // [Hkv*D, d_model] bf16, contiguous
  void* k_out; void* v_out; int64_t o_sb, o_st, o_sh;   // [B, L, Hkv, D] fp8 (one set of strides)
  float* amax;                                          // [2]: max |K|, max |V| (cleared beforehand) or null
  float inv_k, inv_v;                                   // fp32 1/k_scale, 1/v_scale
  int B, L, d_model, Hkv, D;
};
hipError_t launch_kv_bridge(const BridgeArgs& a, hipStream_t s);

}  // namespace hys
