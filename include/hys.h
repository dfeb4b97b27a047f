/*
 * hys.h - C ABI of the HySparse / HySparse2 hybrid-block attention hot path
 *         for AMD Instinct MI355X (gfx950).
 *
 * A hybrid block is one causal full-attention layer followed by N sparse
 * layers that reuse the full layer's KV cache and its top-k indices
 * (QbitAI HySparse article, method section; airebao HySparse2 news, inner
 * KV Reuse paragraph).  The five entry points below are the steps of that
 * block:
 *
 *   hys_full_attn_fwd   - the full layer: exact causal attention that also
 *                         emits importance scores as a byproduct
 *   hys_select_topk     - top-k of each importance row
 *   hys_sparse_attn_fwd - a sparse layer's attention over the selected blocks
 *                         or tokens of the shared KV (HySparse2: plus the
 *                         forced recent window)
 *   hys_swa_gate_fwd    - HySparse's sliding-window branch fused with the
 *                         sigmoid gate that merges it with the sparse branch
 *   hys_decode_step     - one HySparse2 decode step against a long fp8 cache
 *   hys_decode_step_noalloc - the same step on a fixed library-owned scratch
 *                          array, for callers that cannot allocate
 *
 * and one fused form of two of them:
 *
 *   hys_sparse_layer_fwd - a whole HySparse sparse layer (sparse branch,
 *                          window branch and gate) in one pass
 *
 * the HySparse (block-level) decode step:
 *
 *   hys_hysparse_decode_step - full layer with block scores, top-k blocks,
 *                          and every sparse layer (block gather, ring window
 *                          cache with append, gate) for one new query
 *
 * the step that fills HySparse2's shared cache:
 *
 *   hys_kv_bridge_fwd    - KV Bridging: a cross-decoder full layer's K/V
 *                          projected from hidden states into the fp8 cache
 *
 * and the backward pass of the HySparse block (training):
 *
 *   hys_window_attn_fwd  - the window branch alone, with its LSE (the
 *                          forward quantity the sparse layer's backward needs)
 *   hys_full_attn_bwd    - gradients of the full layer's causal attention
 *   hys_sparse_layer_bwd - gradients of one sparse layer (block-sparse
 *                          branch, window branch, gate)
 *
 * Conventions shared by every call
 * --------------------------------
 * Memory:   every tensor pointer is device memory owned by the caller (for
 *           example allocated by PyTorch).  The library allocates nothing,
 *           keeps no pointer after returning and holds no global mutable state
 *           (the one exception: hys_decode_step_noalloc's fixed per-GPU
 *           scratch array and its cached device addresses).
 *           Inputs are only read; outputs are fully overwritten (except
 *           where a call documents an accumulate flag).
 * Streams:  work is enqueued on `stream` (a hipStream_t; NULL = the default
 *           stream) and the call returns without waiting.  Keep every buffer
 *           alive until the stream has finished the work.
 * Layout:   hys_tensor4 describes a [B, T, H, D] tensor (batch, token, head,
 *           head dim) with strides in elements; the head-dim stride must be
 *           1, and D must be 64 or 128.
 * Types:    Q is fp32 or bf16.  K/V are of Q's type, or OCP fp8 e4m3fn when Q
 *           is bf16 (the stored value is decode(byte) * k_scale / v_scale).
 *           Arithmetic is fp32 accumulation on MFMA: fp32 x fp32 for fp32
 *           inputs; bf16 x bf16 otherwise, with softmax probabilities rounded
 *           to bf16 before the P*V product.
 * Workspace:calls that take (ws, ws_bytes) follow one rule: a call with
 *           ws == NULL is a size query - it stores the required size in
 *           *ws_bytes and returns HYS_OK without touching the GPU.  To run,
 *           pass ws != NULL (16-byte aligned device memory) with *ws_bytes at
 *           least the required size; when that size is 0 any non-NULL ws
 *           will do.  hys_sparse_attn_fwd needs no workspace and also runs
 *           with ws == NULL and ws_bytes == NULL.
 * Errors:   arguments are validated before any GPU work.  A failing call
 *           returns a non-zero hys_status, enqueues nothing, and
 *           hys_last_error() returns a message for the calling thread.  It
 *           never aborts and never throws.  Faults inside kernels surface at
 *           the caller's next stream synchronisation.
 * Threads:  the library is stateless; concurrent calls on different streams
 *           are safe (except overlapping hys_decode_step_noalloc calls on one
 *           GPU, which share its scratch array).
 */
#ifndef HYS_H_
#define HYS_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define HYS_ABI_VERSION 6

#if defined(__GNUC__)
#define HYS_API __attribute__((visibility("default")))
#else
#define HYS_API
#endif

typedef enum {
  HYS_OK = 0,
  HYS_ERR_INVALID_ARG = 1,  /* null pointer, bad shape/stride/size, inconsistent tensors */
  HYS_ERR_UNSUPPORTED = 2,  /* valid request outside what the kernels implement */
  HYS_ERR_WORKSPACE = 3,    /* *ws_bytes smaller than required */
  HYS_ERR_HIP = 4,          /* a HIP launch failed */
  HYS_ERR_INTERNAL = 5
} hys_status;

typedef enum { HYS_F32 = 0, HYS_BF16 = 1, HYS_FP8_E4M3 = 2 } hys_dtype;

typedef struct {
  void* ptr;          /* device pointer to element [0,0,0,0] */
  int32_t dtype;      /* hys_dtype */
  int64_t shape[4];   /* [B, T, H, D] */
  int64_t stride[4];  /* element strides; stride[3] must be 1 */
} hys_tensor4;

typedef struct {
  float softmax_scale;  /* multiplies q.k, normally 1/sqrt(D) */
  float k_scale;        /* fp8 K dequantisation scale (1 for fp32/bf16) */
  float v_scale;        /* fp8 V dequantisation scale (1 for fp32/bf16) */
  int32_t causal;       /* must be 1: every layer of the hybrid block attends causally
                           (QbitAI HySparse article, method section); other values
                           return HYS_ERR_UNSUPPORTED */
  int64_t q_offset;     /* absolute position of query row 0 in [0, 2^30): row i of q
                           is position q_offset + i, so a chunk of queries can
                           attend to a longer cache (chunked prefill: the sparse
                           layers reuse the full layer's cache, QbitAI HySparse
                           article, method section).  Needs q_offset + Lq <= Lk.
                           Causal and window ranges use absolute positions; rows
                           of q, o, lse, scores and idx stay relative to the call.
                           The backward calls need 0. */
} hys_attn_params;

typedef enum {
  HYS_SCORE_NONE = 0,
  HYS_SCORE_BLOCK = 1,      /* HySparse: per (query, key block) */
  HYS_SCORE_TILE_TOKEN = 2, /* HySparse2: per (query tile, key token) */
  HYS_SCORE_BLOCK_GROUP = 3 /* per (KV group, query, key block): the max over each KV group's heads */
} hys_score_mode;

typedef struct {
  int32_t mode;  /* hys_score_mode */
  int32_t size;  /* key-block size (BLOCK) or query-tile size (TILE_TOKEN); must be 64 */
} hys_score_params;

typedef struct {
  int32_t granularity;    /* 64: idx holds key-block ids; 1: idx holds token positions */
  int32_t k;              /* entries per idx row */
  int32_t q_tile;         /* queries sharing one idx row: 1 (with granularity 64) or 64 (with granularity 1) */
  int32_t forced_window;  /* granularity 1 only: the recent-token window forced into every query's set (0 = none) */
  int64_t idx_batch_stride;  /* elements between batches of idx */
  int64_t idx_row_stride;    /* elements between idx rows */
  int64_t idx_group_stride;  /* granularity 64: elements between KV groups' index sets; 0 = one set for all */
} hys_sparse_params;

typedef struct {
  float softmax_scale;
  float k_scale, v_scale;
  int32_t topk;    /* tokens selected from the full layer's token scores */
  int32_t window;  /* recent tokens forced into every sparse layer's set */
} hys_decode_params;

/*
 * hys_full_attn_fwd - the full-attention layer of a hybrid block.
 *
 * Computes exact causal scaled dot-product attention
 *   O[b,i,h,:] = sum_{j<=i} softmax_j(S[b,h,i,:]) V[b,j,h/G,:],
 *   S[b,h,i,j] = softmax_scale * k_scale * <Q[b,i,h,:], K[b,j,h/G,:]>,
 * with G = Hq/Hkv query heads per KV head, and LSE[b,h,i] = ln sum_{j<=i} exp(S).
 * As its byproduct it emits importance scores taken from the same logits, the
 * maxima the online softmax already tracks (TechWalker HySparse write-up,
 * paragraph on the modified FlashAttention kernel):
 *   HYS_SCORE_BLOCK:      scores[b,i,c] = max_h max_{j in block c, j<=i} S[b,h,i,j]
 *                         (64-key blocks: airebao HySparse2 news, token-level
 *                         selection paragraph), -inf for blocks after i;
 *                         layout [B, Lq, ceil(Lk/64)] contiguous.
 *   HYS_SCORE_TILE_TOKEN: scores[b,t,j] = max_h max_{i in tile t, i>=j} S[b,h,i,j]
 *                         (token-level importance of HySparse2, one row per
 *                         64-query tile), -inf for keys after the tile;
 *                         layout [B, ceil(Lq/64), Lk] contiguous.
 * The max over heads spans all query heads, so one index set serves every KV
 * head.  HYS_SCORE_BLOCK_GROUP instead keeps one score matrix per KV group,
 *   scores[g,b,i,c] = max_{h in group g} max_{j in block c, j<=i} S[b,h,i,j],
 * layout [Hkv, B, Lq, ceil(Lk/64)] contiguous (per-KV-group selection, an
 * ablation variant of the head reduction; no workspace).
 *
 * q [B, Lq, Hq, D]; k, v [B, Lk, Hkv, D] with p->q_offset + Lq <= Lk: query
 * row i is at position q_offset + i and sees keys j <= q_offset + i (a whole
 * sequence: Lq = Lk, q_offset = 0; a chunk of a longer prefill: its rows and
 * the cache up to its last row).  "i" in the formulas above is that position;
 * rows of o, lse and scores are the call's rows (score tile t = rows 64t ..
 * 64t+63 of the call).
 * o [B, Lq, Hq, D] fp32 or bf16.  lse [B, Hq, Lq] fp32 or NULL.
 * sp may be NULL (no scores); scores must be non-NULL when sp->mode != NONE.
 * Workspace: BLOCK mode with Hkv > 1 needs Hkv * B * Lq * ceil(Lk/64) floats.
 */
HYS_API hys_status hys_full_attn_fwd(const hys_attn_params* p, hys_tensor4 q, hys_tensor4 k, hys_tensor4 v,
                             hys_tensor4 o, float* lse, const hys_score_params* sp, float* scores,
                             void* ws, size_t* ws_bytes, void* stream);

/*
 * hys_select_topk - the k largest entries of each row of a score matrix.
 *
 * The sparse layers attend to the top-k blocks/tokens of the full layer's
 * importance (QbitAI HySparse article, method section; TechWalker write-up).
 * Order: score descending, then column ascending (the lowest column wins a
 * tie).  Only entries > -inf are candidates (NaN and -inf are never chosen).
 * idx[r, 0..k) receives the chosen columns in ascending order, padded with
 * -1; count[r] (if non-NULL) the number chosen.  Selection is exact.
 *
 * scores: rows x cols fp32 with row_stride (elements, >= cols).
 * idx: rows x k int32, contiguous.  Limits: cols < 2^31; k <= 4096.  Rows
 * with more than 32768 columns are selected by a radix select over the whole
 * row that many workgroups share (the row cut into at most 1024 chunks of a
 * multiple of 8192 columns; rows * chunks must stay below 2^22).  Those rows
 * need workspace: per row 5128 + 2 * chunks 32-bit words (row histograms,
 * selection state, per-chunk counts), 4-byte aligned; the call overwrites it.
 */
HYS_API hys_status hys_select_topk(const float* scores, int64_t rows, int64_t cols, int64_t row_stride, int32_t k,
                           int32_t* idx, int32_t* count, void* ws, size_t* ws_bytes, void* stream);

/*
 * hys_select_topk_blocks - block-level selection over token-score rows at a
 * token budget (the block- vs token-level comparison at equal budget:
 * demingchina commentary, section 03).
 *
 * For each row r of the fp32 score matrix (rows x cols, row_stride):
 *   M[r,c] = max_{j in [64c, 64c+64), j < cols} scores[r,j],
 *   the k_blocks highest M[r,:] are chosen by the hys_select_topk rule, and
 *   idx[r,:] (rows x 64*k_blocks int32, contiguous) receives the chosen
 *   blocks' token positions [64c, min(cols, 64c+64)) in ascending block
 *   order, then -1.  The rows can feed hys_sparse_attn_fwd with granularity 1.
 * block must be 64; 1 <= k_blocks <= 32.  Workspace: the block maxima, the
 * block ids and the top-k workspace (query with ws == NULL).
 */
HYS_API hys_status hys_select_topk_blocks(const float* scores, int64_t rows, int64_t cols, int64_t row_stride,
                                          int32_t block, int32_t k_blocks, int32_t* idx, void* ws, size_t* ws_bytes,
                                          void* stream);

/*
 * hys_sparse_attn_fwd - a sparse layer's global attention over the shared KV.
 *
 * The sparse layer attends with its own query q to the full layer's K/V at the
 * selected positions (QbitAI HySparse article, method section; TechWalker
 * write-up: the selected KV blocks form a sparse KV matrix).
 *   granularity 64 (HySparse): idx[b,i,:] lists key-block ids for query i;
 *       J(i) = { j <= i : j/64 in idx[b,i,:] }.
 *   granularity 1, q_tile 64 (HySparse2): idx[b,t,:] lists token positions for
 *       the 64 queries of tile t, and the most recent forced_window tokens are
 *       added (airebao HySparse2 news, forced recent window paragraph):
 *       J(i) = { j in idx[b,i/64,:] : j <= i }  U  [max(0, i-forced_window+1), i].
 * With idx_group_stride != 0 (granularity 64 only), KV group g reads its own
 * index set at idx + g*idx_group_stride (per-KV-group selection):
 *       J_g(i) = { j <= i : j/64 in idx[g,b,i,:] } for the heads of group g.
 * O[b,i,h,:] = softmax over J(i) of S, applied to V; lse[b,h,i] likewise
 * (-inf when J(i) is empty, with O = 0).  Entries < 0 are ignored; entries of
 * a row must be distinct (hys_select_topk guarantees this).
 * q [B, Lq, Hq, D]; k, v [B, Lk, Hkv, D] with p->q_offset + Lq <= Lk: "i"
 * above is the position q_offset + row; idx rows (and tiles) are the call's.
 * o [B, Lq, Hq, D] fp32 or bf16; lse [B, Hq, Lq] fp32 or NULL.
 * Limits: granularity 64 needs k <= 64 and ceil(Lk/64) <= 16384; granularity 1
 * needs k <= 2048 and forced_window <= 1984.  No workspace is used.
 */
HYS_API hys_status hys_sparse_attn_fwd(const hys_attn_params* p, hys_tensor4 q, hys_tensor4 k, hys_tensor4 v,
                               const hys_sparse_params* sp, const int32_t* idx, hys_tensor4 o, float* lse,
                               void* ws, size_t* ws_bytes, void* stream);

/*
 * hys_swa_gate_fwd - HySparse's local branch and the gate.
 *
 * Sliding-window attention of q over the layer's own window cache
 * (k_win, v_win), window [max(0,i-window+1), i] (QbitAI HySparse article:
 * window 128; TechWalker write-up: the most recent 128 tokens, own KV), fused
 * with the sigmoid gate that merges it with the sparse branch:
 *   z = <q[b,i,h,:], gate_w[h,:]> (+ gate_b[h]),  g = 1/(1+exp(-z)),
 *   o = g * o_sparse + (1-g) * O_window,
 * and o = O_window where lse_sparse = -inf (empty sparse set).
 * q [B, Lq, Hq, D]; k_win, v_win [B, Lk, Hkv, D] (p->q_offset + Lq <= Lk; the
 * window is taken at position q_offset + row) of q's type, or fp8 e4m3 with
 * bf16 q (dequantised by p->k_scale, p->v_scale: a gated window over an fp8
 * shared cache, the HySparse2 ablation of the forced window); o_sparse fp32
 * [B, Lq, Hq, D]; lse_sparse [B, Hq, Lq]; gate_w [Hq, D] fp32; gate_b [Hq] or
 * NULL; o [B, Lq, Hq, D] fp32 or bf16.
 */
HYS_API hys_status hys_swa_gate_fwd(const hys_attn_params* p, hys_tensor4 q, hys_tensor4 k_win, hys_tensor4 v_win,
                            int32_t window, hys_tensor4 o_sparse, const float* lse_sparse, const float* gate_w,
                            const float* gate_b, hys_tensor4 o, void* stream);

/*
 * hys_sparse_layer_fwd - one HySparse sparse layer in one pass.
 *
 * Computes what hys_sparse_attn_fwd (granularity 64, q_tile 1) followed by
 * hys_swa_gate_fwd computes (QbitAI HySparse article, method section: the
 * sparse layer's global branch over the selected blocks of the shared KV and
 * its local window branch over its own KV, merged by a sigmoid gate;
 * TechWalker write-up: window 128, independent window KV):
 *   O_sparse = attention of q over J(i) = { j <= i : j/64 in idx[b,i,:] } of k, v
 *   O_window = attention of q over [max(0, i-window+1), i] of k_win, v_win
 *   o = g * O_sparse + (1-g) * O_window,  g = sigmoid(<q, gate_w[h]> (+ gate_b[h])),
 *   o = O_window where J(i) is empty.
 * The sparse branch is never materialised separately: its normalised output
 * is held in o's storage type between the branches (so with a bf16 o it is
 * rounded to bf16 before the gate; with fp32 o the result matches the
 * two-call form up to fp32 rounding).
 * q [B, Lq, Hq, D] bf16 or fp32; k, v, k_win, v_win [B, Lk, Hkv, D] of q's
 * type (p->q_offset + Lq <= Lk, positions as for hys_sparse_attn_fwd), the
 * window tensors with the same strides as k and v; idx and sp as for
 * hys_sparse_attn_fwd with granularity 64 (k <= 64; per-KV-group index sets
 * through idx_group_stride as there); gate_w [Hq, D] fp32;
 * gate_b [Hq] fp32 or NULL; o [B, Lq, Hq, D] fp32 or bf16.  p->k_scale and
 * p->v_scale must be 1.  No workspace.
 */
HYS_API hys_status hys_sparse_layer_fwd(const hys_attn_params* p, hys_tensor4 q, hys_tensor4 k, hys_tensor4 v,
                                const hys_sparse_params* sp, const int32_t* idx, hys_tensor4 k_win,
                                hys_tensor4 v_win, int32_t window, const float* gate_w, const float* gate_b,
                                hys_tensor4 o, void* stream);

/*
 * hys_decode_step - one HySparse2 decode step (airebao HySparse2 news:
 * token-level selection, forced recent window, MQA, 1M-token FP8 cache).
 *
 * For each sequence b with valid cache length n = cache_len[b] (the cache
 * already holds the new token at position n-1):
 *   full layer:   o_full[b,0,h,:] = attention of q_full[b,0,h,:] over keys [0, n);
 *                 token_scores[b,j] = max_h S[b,h,j] for j < n, -inf for j >= n;
 *   selection:    idx[b,:] = top-topk of token_scores[b,:] (ascending, -1 padded);
 *   sparse layers l = 0..n_sparse-1:
 *                 o_sparse[l][b,0,h,:] = attention of q_sparse[l][b,0,h,:] over
 *                 idx[b,:] U [max(0, n-window), n-1], all over the same cache.
 * q_full and q_sparse[l]: [B, 1, Hq, D] bf16, all q_sparse with equal strides.
 * k_cache, v_cache: [B, Nmax, 1, D] fp8 e4m3fn or bf16 (MQA: one KV head).
 * cache_len: HOST array of B lengths, 1 <= n <= Nmax.
 * o_full, o_sparse[l]: [B, 1, Hq, D] fp32 or bf16 (all of one type).
 * token_scores: [B, Nmax] fp32 (required).  idx: [B, topk] int32.
 * Limits: Hq <= 64, B <= 64, n_sparse <= 16, topk <= 2048.
 * Workspace: split partials, the top-k's row histograms and counts (query with ws == NULL).
 */
HYS_API hys_status hys_decode_step(const hys_decode_params* p, hys_tensor4 q_full, hys_tensor4 k_cache,
                           hys_tensor4 v_cache, const int64_t* cache_len, hys_tensor4 o_full, float* token_scores,
                           int32_t* idx, int32_t n_sparse, const hys_tensor4* q_sparse,
                           const hys_tensor4* o_sparse, void* ws, size_t* ws_bytes, void* stream);

/* Size of the fixed device scratch array behind hys_decode_step_noalloc. */
#define HYS_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

/*
 * hys_decode_step_noalloc - hys_decode_step for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, and
 * harnesses that forbid hipMalloc.  Same arguments, outputs and kernels as
 * hys_decode_step, without (ws, ws_bytes): the workspace is a fixed array
 * of HYS_NOALLOC_SCRATCH_BYTES (64 MiB) of device memory inside the library,
 * one copy per GPU, held until the process ends.  The call allocates and
 * frees nothing (no hipMalloc, hipFree or allocating library routine).
 * Limit: a step whose workspace (the size hys_decode_step reports for the
 * same arguments) exceeds the array returns HYS_ERR_WORKSPACE before any GPU
 * work; the 1,048,576-token, 4-sequence, 11-layer step needs about 30 MiB.
 * Set-up: the first call on a device looks up that device's copy of the
 * array (hipGetSymbolAddress, with the device current) and keeps its address.
 * Sharing: every call on one GPU uses that GPU's one array, and nothing in
 * it has to start cleared (each step writes every scratch value before
 * reading it).  Calls that overlap in time on one GPU (other threads, other
 * streams) race on the array: serialise them, e.g. on one stream.
 */
HYS_API hys_status hys_decode_step_noalloc(const hys_decode_params* p, hys_tensor4 q_full, hys_tensor4 k_cache,
                                           hys_tensor4 v_cache, const int64_t* cache_len, hys_tensor4 o_full,
                                           float* token_scores, int32_t* idx, int32_t n_sparse,
                                           const hys_tensor4* q_sparse, const hys_tensor4* o_sparse, void* stream);

typedef struct {
  float softmax_scale;
  int32_t topk;   /* key blocks selected from the full layer's block scores (1..64) */
  int32_t block;  /* key-block size; must be 64 */
} hys_hs_decode_params;

/*
 * hys_hysparse_decode_step - one HySparse decode step (block-level selection
 * with a gated sliding-window branch; QbitAI HySparse article, method section;
 * TechWalker write-up: 64-token blocks, window 128 over the layer's own K/V).
 *
 * For each sequence b with valid cache length n = cache_len[b] (the shared
 * cache already holds the new token at position n-1):
 *   full layer:   o_full[b,0,h,:] = attention of q_full[b,0,h,:] over keys
 *                 [0, n) of KV head h/G (G = Hq/Hkv);
 *                 block_scores[b,c] = max_h max_{j in block c, j < n} S[b,h,j]
 *                 (-inf for blocks with no key below n);
 *   selection:    idx[b,:] = top-topk of block_scores[b,:] (block ids,
 *                 ascending, -1 padded; the hys_select_topk rule);
 *   sparse layers l = 0..n_sparse-1, each with a ring window cache of W slots
 *   (token t in slot t mod W):
 *                 the new token's window K/V k_win_new[l], v_win_new[l] is
 *                 written into slot (n-1) mod W of k_ring[l], v_ring[l];
 *                 O_sp = attention of q_sparse[l] over { j < n : j/64 in idx[b,:] }
 *                 of the shared cache; O_w = attention over the window tokens
 *                 [max(0, n-W), n-1] of the ring;
 *                 o_sparse[l] = g O_sp + (1-g) O_w, g = sigmoid(<q, gate_w[l][h,:]>),
 *                 and o_sparse[l] = O_w where the selected set is empty.
 * q_full, q_sparse[l]: [B, 1, Hq, D] bf16 (all q_sparse with equal strides).
 * k_cache, v_cache: [B, Nmax, Hkv, D] bf16.  cache_len: HOST array of B
 * lengths, 1 <= n <= Nmax.  o_full, o_sparse[l]: [B, 1, Hq, D] fp32 or bf16
 * (all o_sparse of one type and strides).  block_scores: [B, ceil(Nmax/64)]
 * fp32, contiguous.  idx: [B, topk] int32.
 * k_win_new[l], v_win_new[l]: [B, 1, Hkv, D] bf16; k_ring[l], v_ring[l]:
 * [B, W, Hkv, D] bf16, updated in place; every new and ring tensor with one
 * set of strides.  gate_w[l]: [Hq, D] fp32, contiguous.  The window length
 * is W = k_ring[0].shape[1].
 * Limits: Hq = Hkv*G with G in {1, 2, 4, 8, 16}, B <= 64, n_sparse <= 16,
 * topk <= 64.
 * Workspace: per-KV-head token scores and split partials, the top-k workspace
 * (query with ws == NULL).
 */
HYS_API hys_status hys_hysparse_decode_step(const hys_hs_decode_params* p, hys_tensor4 q_full, hys_tensor4 k_cache,
                                            hys_tensor4 v_cache, const int64_t* cache_len, hys_tensor4 o_full,
                                            float* block_scores, int32_t* idx, int32_t n_sparse,
                                            const hys_tensor4* q_sparse, const hys_tensor4* k_win_new,
                                            const hys_tensor4* v_win_new, const hys_tensor4* k_ring,
                                            const hys_tensor4* v_ring, const float* const* gate_w,
                                            const hys_tensor4* o_sparse, void* ws, size_t* ws_bytes, void* stream);

typedef struct {
  float k_scale;  /* K cache quantisation scale: the stored code is e4m3(K / k_scale) */
  float v_scale;  /* V cache quantisation scale */
} hys_bridge_params;

/*
 * hys_kv_bridge_fwd - HySparse2's KV Bridging projection (airebao HySparse2
 * news, outer KV Bridging paragraph; demingchina commentary, section 02).
 *
 * The cross-decoder's full-attention layers take their K and V from the
 * hidden states of the self-decoder's full-attention layer, so the shared
 * MQA cache is written once, in FP8 (airebao key-data table):
 *   K[b,t,:] = h[b,t,:] W_k^T,  V[b,t,:] = h[b,t,:] W_v^T   (no bias),
 *   k_cache[b,t,g,d] = e4m3(K[b,t,g*D+d] / k_scale),  v_cache likewise,
 * with e4m3 the OCP e4m3fn code of the value rounded to nearest (ties to
 * even) and saturated at +-448; K and V are accumulated in fp32 from bf16
 * products and multiplied by the fp32 reciprocal of the scale.  Infinite
 * projections saturate; the codes of NaN projections are unspecified.
 * amax, when not NULL, receives max |K| and max |V| over the fp32
 * projections (0 when B*L = 0), so that a caller can set the next scales
 * (scale = amax / 448); it is overwritten, not accumulated.
 *
 * h: [B, L, 1, d_model] bf16, d_model a multiple of 64 in [64, 32768],
 *    token and batch strides multiples of 8 elements.
 * w_k, w_v: [Hkv*D, d_model] bf16, contiguous ([out, in] layout), 16-byte
 *    aligned device memory.
 * k_cache, v_cache: [B, L, Hkv, D] fp8 e4m3fn with identical shapes and
 *    strides, D in {64, 128} and Hkv*D a multiple of 128.  Pass a view to
 *    write positions [t0, t0+L) of a longer cache.
 * With L = 0 only amax is written, and the h and cache pointers may be NULL.
 * No workspace.
 */
HYS_API hys_status hys_kv_bridge_fwd(const hys_bridge_params* p, hys_tensor4 h, const void* w_k, const void* w_v,
                                     hys_tensor4 k_cache, hys_tensor4 v_cache, float* amax, void* stream);

/*
 * Backward pass of the HySparse block.
 *
 * The pages say the hybrid structure is trained directly (QbitAI HySparse
 * article, opening summary; demingchina commentary, section 06).  The
 * selection is held fixed (top-k passes no gradient), so every branch's
 * gradients are those of softmax attention over its visible set J(i):
 *   P = softmax_J(S), S = scale * q k^T:  dV = P^T dO,  dS = P * (dO v^T - rowsum(dO * O)),
 *   dQ = scale * dS k,  dK = scale * dS^T q,
 * summed over the G query heads of each KV head.  All gradients are fp32;
 * q, k, v and their window counterparts must be bf16 with p->k_scale =
 * p->v_scale = 1.  P and dS are rounded to bf16 before their products (as P
 * is in the forward).  dK/dV of the shared cache can accumulate (accumulate_kv
 * = 1 adds into dk, dv instead of overwriting them) so that the full layer and
 * every sparse layer of a block sum into one buffer, in call order.
 */

/*
 * hys_window_attn_fwd - sliding-window attention alone: O and LSE of the
 * window branch of hys_swa_gate_fwd, without the gate (window [max(0,
 * i-window+1), i] over k_win, v_win).  q, k_win, v_win as for
 * hys_swa_gate_fwd; o [B, L, Hq, D] fp32 or bf16; lse [B, Hq, L] fp32
 * (natural log) or NULL.  No workspace.
 */
HYS_API hys_status hys_window_attn_fwd(const hys_attn_params* p, hys_tensor4 q, hys_tensor4 k_win, hys_tensor4 v_win,
                                       int32_t window, hys_tensor4 o, float* lse, void* stream);

/*
 * hys_full_attn_bwd - gradients of the full layer's causal attention.
 *
 * q [B, L, Hq, D], k, v [B, L, Hkv, D] bf16 (k and v with one set of
 * strides); o (fp32 or bf16) and lse [B, Hq, L] from hys_full_attn_fwd; d_o
 * [B, L, Hq, D] bf16, the upstream gradient.  dq [B, L, Hq, D] fp32 is
 * overwritten; dk, dv [B, L, Hkv, D] fp32 (one set of strides) are
 * overwritten, or added to with accumulate_kv = 1.  Workspace (query with
 * ws == NULL): rowsum(dO * O) (4*B*Hq*L bytes) and, for L above 2048, the
 * dK/dV row splits' partial sums (up to 16 copies of dk and dv) with their
 * flags.
 */
HYS_API hys_status hys_full_attn_bwd(const hys_attn_params* p, hys_tensor4 q, hys_tensor4 k, hys_tensor4 v,
                                     hys_tensor4 o, const float* lse, hys_tensor4 d_o, hys_tensor4 dq, hys_tensor4 dk,
                                     hys_tensor4 dv, int32_t accumulate_kv, void* ws, size_t* ws_bytes, void* stream);

/*
 * hys_sparse_layer_bwd - gradients of one HySparse sparse layer
 * (hys_sparse_layer_fwd's computation: block-sparse branch over the shared
 * k, v at the selected blocks, window branch over k_win, v_win, sigmoid gate).
 *
 * With g = sigmoid(<q, gate_w[h]> + gate_b[h]) and o = g O_sp + (1-g) O_w
 * (o = O_w where lse_sparse = -inf), the upstream gradient d_o splits into
 * g d_o for the sparse branch and (1-g) d_o for the window branch, and the
 * gate adds dz = g (1-g) <d_o, O_sp - O_w> to the layer:
 *   dq += dz gate_w[h],   dgate_w[h] = sum over (b, i) of dz q[b,i,h,:],
 *   dgate_b[h] = sum over (b, i) of dz.
 * Inputs: q bf16; k, v (shared) and k_win, v_win bf16 of equal shapes (k and
 * v with one set of strides, k_win and v_win with one set); sp and idx as
 * for hys_sparse_attn_fwd with granularity 64, q_tile 1, no forced window
 * (idx_group_stride for per-KV-group sets); o_sparse, lse_sparse from
 * hys_sparse_attn_fwd and o_win, lse_win from hys_window_attn_fwd (outputs
 * fp32 or bf16, lse [B, Hq, L]); gate_w [Hq, D] fp32, gate_b [Hq] or NULL;
 * d_o [B, L, Hq, D] fp32 or bf16.
 * Outputs (fp32): dq [B, L, Hq, D] overwritten; dk, dv [B, L, Hkv, D] (one
 * set of strides) overwritten or, with accumulate_kv = 1, added to; dk_win,
 * dv_win [B, L, Hkv, D] (one set of strides) overwritten; dgate_w [Hq, D]
 * contiguous, overwritten; dgate_b [Hq] (the bias's gradient, the row sum of
 * dz) overwritten, or NULL when not wanted.  Workspace (query with ws == NULL): the two branch
 * gradients in bf16 (2*B*L*Hq*D bytes each), three [B, Hq, L] fp32 arrays,
 * the selection bitmaps, the gate's partial sums and, for L above 2048, the
 * shared dK/dV row splits' partial sums (up to 16 copies of dk and dv).
 */
HYS_API hys_status hys_sparse_layer_bwd(const hys_attn_params* p, hys_tensor4 q, hys_tensor4 k, hys_tensor4 v,
                                        const hys_sparse_params* sp, const int32_t* idx, hys_tensor4 k_win,
                                        hys_tensor4 v_win, int32_t window, const float* gate_w, const float* gate_b,
                                        hys_tensor4 o_sparse, const float* lse_sparse, hys_tensor4 o_win,
                                        const float* lse_win, hys_tensor4 d_o, hys_tensor4 dq, hys_tensor4 dk,
                                        hys_tensor4 dv, int32_t accumulate_kv, hys_tensor4 dk_win, hys_tensor4 dv_win,
                                        float* dgate_w, float* dgate_b, void* ws, size_t* ws_bytes, void* stream);

/* Message for the calling thread's last non-OK status ("" if none). */
HYS_API const char* hys_last_error(void);
/* Static name of a status code. */
HYS_API const char* hys_status_string(hys_status s);
/* HYS_ABI_VERSION of the built library. */
HYS_API int hys_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* HYS_H_ */
