"""Plain fp64 definitions of every step of the HySparse / HySparse2 hybrid block.

TEST INFRASTRUCTURE ONLY (see the package header).

Notation (one sequence at a time; batch is an outer loop):
  q  [L, Hq, D]   query of a layer, float64
  k, v [L, Hkv, D] the full-attention layer's keys / values, float64
  G = Hq / Hkv;   query head h reads KV head h // G
  scale = 1/sqrt(D); positions are 0-based; key j is visible to query i iff j <= i.

Every function evaluates only the query rows it is asked for (`rows`), so the
same definitions serve tiny exhaustive checks and sampled rows of the
full-size workloads.  No blocking, fusion or reordering is used beyond
computing rows independently: each row's logits are formed explicitly and
passed through an explicit softmax.

Sources (the pages; each citation below names the page and the passage):
  [QbitAI]     = QbitAI HySparse article, method section (the full-attention
               layer does the selection and keeps the cache)
  [TechWalker] = TechWalker HySparse write-up, paragraphs on the modified
               FlashAttention kernel and on the sparse layers
  [airebao]    = airebao HySparse2 news, paragraphs "core mechanism", "inner
               KV Reuse", "token-level selection", "forced recent window",
               "MQA detail" and the key-data table
  [deming]     = demingchina HySparse2 commentary, sections 03 and 05
A bracketed tag in a docstring abbreviates that page; the passage is named
next to it.
"""
from __future__ import annotations

from typing import Dict, Iterable, List, Optional, Sequence

import numpy as np

NEG_INF = -np.inf


# ----------------------------------------------------------------------------
# logits and softmax attention
# ----------------------------------------------------------------------------

def logits(q_rows: np.ndarray, k: np.ndarray, scale: float, G: int) -> np.ndarray:
    """Scaled dot-product logits S[h, r, j] = scale * <q_rows[r,h,:], k[j,h//G,:]>.

    The full layer computes standard scaled dot-product attention [TechWalker,
    implementation paragraph]; query head h shares KV head h // G (GQA / MQA,
    [airebao] MQA detail).
    """
    R, Hq, _ = q_rows.shape
    out = np.empty((Hq, R, k.shape[0]), dtype=np.float64)
    for h in range(Hq):
        out[h] = scale * (q_rows[:, h, :] @ k[:, h // G, :].T)
    return out


def attend(S: np.ndarray, v: np.ndarray, G: int):
    """Softmax over the unmasked entries of each logit row, applied to V.

    S[h, r, j] holds logits with excluded keys set to -inf.  For each row:
      m = max_j S,  P_j = exp(S_j - m) / sum_j exp(S_j - m),  O = sum_j P_j V_j,
      LSE = m + ln sum_j exp(S_j - m)   (natural log).
    A row with no visible key returns O = 0 and LSE = -inf.
    Returns O [R, Hq, D] and LSE [Hq, R].
    """
    Hq, R, _ = S.shape
    D = v.shape[-1]
    m = S.max(axis=2)
    live = np.isfinite(m)
    m0 = np.where(live, m, 0.0)
    P = np.exp(S - m0[:, :, None])
    l = P.sum(axis=2)
    l1 = np.where(live, l, 1.0)
    O = np.zeros((R, Hq, D), dtype=np.float64)
    for h in range(Hq):
        num = P[h] @ v[:, h // G, :]
        O[:, h, :] = np.where(live[h][:, None], num / l1[h][:, None], 0.0)
    lse = np.where(live, m0 + np.log(l1), NEG_INF)
    return O, lse


def _rows(rows, L) -> np.ndarray:
    return np.arange(L, dtype=np.int64) if rows is None else np.asarray(rows, dtype=np.int64)


def _causal_allowed(rows: np.ndarray, Lk: int) -> np.ndarray:
    j = np.arange(Lk, dtype=np.int64)
    return j[None, :] <= rows[:, None]


# ----------------------------------------------------------------------------
# a1: full causal attention of the full layer
# ----------------------------------------------------------------------------

def full_attention(q, k, v, scale, rows=None):
    """Exact causal attention of the full layer for the query rows `rows`.

    [QbitAI]: the full-attention layer of each hybrid block computes exact
    attention; [TechWalker]: the full layer runs standard scaled dot-product
    attention.  Returns O [R, Hq, D], LSE [Hq, R].
    """
    L, Hq, _ = q.shape
    G = Hq // k.shape[1]
    rows = _rows(rows, L)
    S = logits(q[rows], k, scale, G)
    S[:, ~_causal_allowed(rows, k.shape[0])] = NEG_INF
    return attend(S, v, G)


# ----------------------------------------------------------------------------
# a2: importance scores emitted by the full layer
# ----------------------------------------------------------------------------

def block_scores(q, k, scale, block, rows=None):
    """HySparse block importance M[i, c] = max_h max_{j in block c, j <= i} S[h, i, j].

    [TechWalker]: the full layer's FlashAttention kernel reuses the row-wise
    maximum logits of its online softmax to emit block-level maximum
    attention scores; the blocks are 64 tokens ([airebao] token-level
    selection paragraph; [deming] section 03).  The max is taken over all
    query heads so one index set per query serves every KV head, and over
    causal entries only; wholly future blocks score -inf.
    Returns M [R, ceil(L/block)].
    """
    L, Hq, _ = q.shape
    G = Hq // k.shape[1]
    Lk = k.shape[0]
    rows = _rows(rows, L)
    S = logits(q[rows], k, scale, G)
    S[:, ~_causal_allowed(rows, Lk)] = NEG_INF
    Sh = S.max(axis=0)                              # [R, Lk] max over heads
    nblk = (Lk + block - 1) // block
    pad = np.full((len(rows), nblk * block), NEG_INF)
    pad[:, :Lk] = Sh
    return pad.reshape(len(rows), nblk, block).max(axis=2)


def block_scores_per_group(q, k, scale, block, rows=None):
    """Per-KV-group block importance, the ablation of the head reduction (R1).

    M[g, i, c] = max over the query heads h of KV group g (h // G == g) of
    max_{j in block c, j <= i} S[h, i, j]: each KV group selects for itself
    instead of one index set serving every group.  Returns [Hkv, R, nblk].
    """
    L, Hq, _ = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    Lk = k.shape[0]
    rows = _rows(rows, L)
    S = logits(q[rows], k, scale, G)
    S[:, ~_causal_allowed(rows, Lk)] = NEG_INF
    nblk = (Lk + block - 1) // block
    out = np.empty((Hkv, len(rows), nblk))
    for g in range(Hkv):
        Sg = S[g * G:(g + 1) * G].max(axis=0)       # [R, Lk] max over the group's heads
        pad = np.full((len(rows), nblk * block), NEG_INF)
        pad[:, :Lk] = Sg
        out[g] = pad.reshape(len(rows), nblk, block).max(axis=2)
    return out


def tile_token_scores(q, k, scale, tile, tiles=None):
    """HySparse2 token importance T[t, j] = max_h max_{i in tile t, i >= j} S[h, i, j].

    [airebao] token-level selection: HySparse2 scores single tokens instead of
    64-token blocks; the per-tile reading (one score row and one index set per
    64-query tile) is this build's plain reading of how a prefill kernel with
    64-row tiles emits token-level importance.  Keys after the tile's last
    query score -inf.  Returns T [len(tiles), Lk].
    """
    L, Hq, _ = q.shape
    G = Hq // k.shape[1]
    Lk = k.shape[0]
    ntile = (L + tile - 1) // tile
    tiles = np.arange(ntile) if tiles is None else np.asarray(tiles, dtype=np.int64)
    out = np.empty((len(tiles), Lk), dtype=np.float64)
    for n, t in enumerate(tiles):
        rows = np.arange(t * tile, min(L, (t + 1) * tile), dtype=np.int64)
        S = logits(q[rows], k, scale, G)
        S[:, ~_causal_allowed(rows, Lk)] = NEG_INF
        out[n] = S.max(axis=(0, 1))
    return out


# ----------------------------------------------------------------------------
# a3: top-k selection
# ----------------------------------------------------------------------------

def topk_select(x, k):
    """Indices of the k highest scores of one row.

    [QbitAI] / [TechWalker]: a TopK over the full layer's importance scores
    picks the blocks (or tokens) the sparse layers attend to.  The pages fix no
    tie rule; here the order is (score descending, index ascending), so the
    lowest index wins a tie.  Only entries > -inf are candidates (NaN and
    -inf are never chosen).  Output: the chosen indices in ascending order,
    padded with -1 to length k, and the number chosen.
    """
    x = np.asarray(x, dtype=np.float64)
    k = int(k)
    cand = np.nonzero(x > NEG_INF)[0]
    order = np.lexsort((cand, -x[cand]))
    chosen = np.sort(cand[order[:k]])
    out = np.full(k, -1, dtype=np.int64)
    out[:len(chosen)] = chosen
    return out, len(chosen)


def topk_rows(scores, k):
    """topk_select applied to every row of a 2-D score array."""
    scores = np.asarray(scores)
    idx = np.full((scores.shape[0], int(k)), -1, dtype=np.int64)
    cnt = np.zeros(scores.shape[0], dtype=np.int64)
    for r in range(scores.shape[0]):
        idx[r], cnt[r] = topk_select(scores[r], k)
    return idx, cnt


# ----------------------------------------------------------------------------
# a4: sparse attention over the shared KV
# ----------------------------------------------------------------------------

def sparse_block_attention(q, k, v, scale, sel, block, rows=None):
    """HySparse global branch: attention over the selected 64-token blocks.

    [QbitAI]: each sparse layer's global branch attends over the shared KV
    cache at the full layer's TopK block indices; [TechWalker]: the selected
    KV blocks are concatenated into a sparse KV matrix attended with the
    layer's own query.  J(i) = {j <= i : j // block in sel_i}.
    `sel` [R, kb] holds block ids for the rows in `rows` (-1 = unused).
    An empty J gives O = 0 and LSE = -inf.
    """
    L, Hq, _ = q.shape
    G = Hq // k.shape[1]
    Lk = k.shape[0]
    rows = _rows(rows, L)
    allowed = np.zeros((len(rows), Lk), dtype=bool)
    for r in range(len(rows)):
        for c in np.asarray(sel[r]):
            if c >= 0:
                allowed[r, c * block:(c + 1) * block] = True
    allowed &= _causal_allowed(rows, Lk)
    S = logits(q[rows], k, scale, G)
    S[:, ~allowed] = NEG_INF
    return attend(S, v, G)


def sparse_block_attention_grouped(q, k, v, scale, sel_g, block, rows=None):
    """Block-sparse branch with one index set per KV group (per-group variant):
    head h attends J_{h//G}(i) = {j <= i : j // block in sel_g[h // G, i]}.
    `sel_g` [Hkv, R, kb] holds block ids for the rows in `rows` (-1 = unused)."""
    L, Hq, _ = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    Lk = k.shape[0]
    rows = _rows(rows, L)
    causal = _causal_allowed(rows, Lk)
    S = logits(q[rows], k, scale, G)
    for g in range(Hkv):
        allowed = np.zeros((len(rows), Lk), dtype=bool)
        for r in range(len(rows)):
            for c in np.asarray(sel_g[g][r]):
                if c >= 0:
                    allowed[r, c * block:(c + 1) * block] = True
        allowed &= causal
        S[g * G:(g + 1) * G][:, ~allowed] = NEG_INF
    return attend(S, v, G)


def sparse_token_attention(q, k, v, scale, sel_tiles, tile, window, rows=None):
    """HySparse2 sparse layer: selected tokens united with a forced recent window.

    airebao HySparse2 news, token-level selection and forced recent window
    paragraphs: a sparse layer attends to individually chosen tokens, and the
    128 newest tokens are always added to that choice; the window therefore
    reads the same cache as the chosen tokens and no second (window) branch
    exists (demingchina HySparse2 commentary, section 03).
    J(i) = {j in sel_{i // tile} : j <= i}  U  [max(0, i-window+1), i]
    (a set union: a token in both counts once).  `sel_tiles` [ntile, kt].
    """
    L, Hq, _ = q.shape
    G = Hq // k.shape[1]
    Lk = k.shape[0]
    rows = _rows(rows, L)
    allowed = np.zeros((len(rows), Lk), dtype=bool)
    for r, i in enumerate(rows):
        s = np.asarray(sel_tiles[i // tile])
        s = s[s >= 0]
        allowed[r, s] = True
        allowed[r, max(0, i - window + 1):i + 1] = True
    allowed &= _causal_allowed(rows, Lk)
    S = logits(q[rows], k, scale, G)
    S[:, ~allowed] = NEG_INF
    return attend(S, v, G)


# ----------------------------------------------------------------------------
# a5: sliding-window branch and sigmoid gate (HySparse)
# ----------------------------------------------------------------------------

def window_attention(q, kw, vw, scale, window, rows=None):
    """Sliding-window branch over the layer's own small KV cache.

    [QbitAI]: the local branch keeps its own window KV (default window 128);
    [TechWalker]: it models the most recent 128 tokens.  Reading: the window
    of query i is [max(0, i-window+1), i], 128 keys including i itself.
    """
    L, Hq, _ = q.shape
    G = Hq // kw.shape[1]
    Lk = kw.shape[0]
    rows = _rows(rows, L)
    j = np.arange(Lk, dtype=np.int64)
    allowed = (j[None, :] <= rows[:, None]) & (j[None, :] >= rows[:, None] - window + 1)
    S = logits(q[rows], kw, scale, G)
    S[:, ~allowed] = NEG_INF
    return attend(S, vw, G)


def gate_merge(q_rows, gate_w, o_sp, lse_sp, o_w, gate_b=None):
    """Sigmoid-gated fusion of the global (sparse) and local (window) branches.

    [QbitAI]: the two branch outputs are fused by a lightweight sigmoid gate;
    [TechWalker]: both branches use the same query and are weighted by a
    sigmoid gate.  Reading: one scalar gate per (token, head),
      g = 1 / (1 + exp(-(<q[i,h,:], w[h,:]> + b[h]))),  O = g * O_sp + (1 - g) * O_w,
    with the optional per-head bias b absent (0) in the plain reading, and
    when the sparse set is empty (LSE_sp = -inf) the branch is absent: O = O_w.
    q_rows [R, Hq, D]; gate_w [Hq, D]; o_sp, o_w [R, Hq, D]; lse_sp [Hq, R]; gate_b [Hq] or None.
    """
    z = np.einsum("rhd,hd->rh", q_rows, gate_w)
    if gate_b is not None:
        z = z + np.asarray(gate_b)[None, :]
    g = 1.0 / (1.0 + np.exp(-z))
    out = g[:, :, None] * o_sp + (1.0 - g)[:, :, None] * o_w
    empty = ~np.isfinite(np.asarray(lse_sp).T)
    out[empty] = o_w[empty]
    return out


# ----------------------------------------------------------------------------
# a6: HySparse2 decode step
# ----------------------------------------------------------------------------

def decode_full(qd, kc, vc, scale, n):
    """Full layer at decode: one query at position n-1 against keys [0, n).

    [airebao] key-data table: the decode analysis is at 1M tokens with an FP8
    KV cache; [QbitAI] background: decoding keeps the whole KV cache, so
    bandwidth dominates.  qd [Hq, D]; kc, vc [N, Hkv, D].
    Returns o [Hq, D], lse [Hq], token scores s[j] = max_h S[h, j] for j < n.
    """
    Hq = qd.shape[0]
    G = Hq // kc.shape[1]
    S = logits(qd[None], kc[:n], scale, G)         # [Hq, 1, n]
    O, lse = attend(S, vc[:n], G)
    return O[0], lse[:, 0], S[:, 0, :].max(axis=0)


def decode_sparse(qd, kc, vc, scale, n, sel, window):
    """Sparse layer at decode: J = sel U [n-window, n-1] over the shared cache."""
    Hq = qd.shape[0]
    G = Hq // kc.shape[1]
    allowed = np.zeros(n, dtype=bool)
    s = np.asarray(sel)
    s = s[(s >= 0) & (s < n)]
    allowed[s] = True
    allowed[max(0, n - window):n] = True
    S = logits(qd[None], kc[:n], scale, G)
    S[:, 0, ~allowed] = NEG_INF
    O, lse = attend(S, vc[:n], G)
    return O[0], lse[:, 0]


# ----------------------------------------------------------------------------
# the hybrid block (one full layer feeding N sparse layers)
# ----------------------------------------------------------------------------

def hysparse_block(q_layers, k, v, kw_layers, vw_layers, gate_layers, scale,
                   block, topk, window, rows=None):
    """One HySparse hybrid block for the query rows `rows` (one sequence).

    [QbitAI]: a hybrid block is 1 full-attention layer + N sparse layers that
    reuse the full layer's important-token indices and KV cache; each sparse
    layer has a block-sparse global branch and a window branch fused by a
    sigmoid gate.  q_layers[0] is the full layer's query, q_layers[l] (l>=1)
    the l-th sparse layer's.  The same `sel` and the same K/V serve every
    sparse layer.
    """
    q0 = q_layers[0]
    L = q0.shape[0]
    rows = _rows(rows, L)
    o_full, lse = full_attention(q0, k, v, scale, rows)
    sc = block_scores(q0, k, scale, block, rows)
    sel, cnt = topk_rows(sc, topk)
    outs = []
    for l in range(1, len(q_layers)):
        ql = q_layers[l]
        o_sp, lse_sp = sparse_block_attention(ql, k, v, scale, sel, block, rows)
        o_w, _ = window_attention(ql, kw_layers[l - 1], vw_layers[l - 1], scale, window, rows)
        outs.append(gate_merge(ql[rows], gate_layers[l - 1], o_sp, lse_sp, o_w))
    return dict(o_full=o_full, lse=lse, scores=sc, sel=sel, count=cnt, o_layers=outs)


def hysparse2_block(q_layers, k, v, scale, tile, topk, window, tiles=None):
    """One HySparse2 hybrid block (prefill), evaluated for whole query tiles.

    [airebao] inner KV Reuse: the sparse layers reuse the full layer's KV
    cache and top-k indices; selection is token-level (top-1024) and the
    recent window is forced into the selected set.
    """
    q0 = q_layers[0]
    L = q0.shape[0]
    ntile = (L + tile - 1) // tile
    tiles = np.arange(ntile) if tiles is None else np.asarray(tiles, dtype=np.int64)
    rows = np.concatenate([np.arange(t * tile, min(L, (t + 1) * tile)) for t in tiles]).astype(np.int64)
    o_full, lse = full_attention(q0, k, v, scale, rows)
    T = tile_token_scores(q0, k, scale, tile, tiles)
    sel_t, cnt = topk_rows(T, topk)
    sel_full = np.full((ntile, int(topk)), -1, dtype=np.int64)
    sel_full[tiles] = sel_t
    outs = []
    for l in range(1, len(q_layers)):
        o, _ = sparse_token_attention(q_layers[l], k, v, scale, sel_full, tile, window, rows)
        outs.append(o)
    return dict(rows=rows, o_full=o_full, lse=lse, scores=T, sel=sel_t, count=cnt, o_layers=outs)


def decode_step(q_full, kc, vc, scale, n, q_sparse, topk, window):
    """HySparse2 decode step for one sequence of valid length n.

    Full layer (attention + token scores) -> top-k over the n scores ->
    each sparse layer attends over the selected tokens united with the
    recent window, all over the same cache.
    """
    o_full, lse, s = decode_full(q_full, kc, vc, scale, n)
    sel, cnt = topk_select(s, topk)
    outs = [decode_sparse(ql, kc, vc, scale, n, sel, window)[0] for ql in q_sparse]
    return dict(o_full=o_full, lse=lse, scores=s, sel=sel, count=cnt, o_layers=outs)


# ----------------------------------------------------------------------------
# ablation variants (switches on the HySparse2 block)
# ----------------------------------------------------------------------------

def hysparse2_gated_window_layer(q, k, v, scale, sel_tiles, tile, window, gate_w, rows=None):
    """HySparse2 sparse layer with a gated sliding-window branch instead of the
    forced recent window (the ablation of [airebao] forced recent window
    paragraph, where a gated SWA is compared with forcing the window into the
    selected set).  Reading: the window branch covers the same 128 recent
    tokens of the shared cache, and the two branches are fused by the HySparse
    sigmoid gate:  o = g * O(sel) + (1 - g) * O(window), o = O(window) when the
    selected set is empty.
    """
    L = q.shape[0]
    rows = _rows(rows, L)
    o_sp, lse_sp = sparse_token_attention(q, k, v, scale, sel_tiles, tile, 0, rows)
    o_w, _ = window_attention(q, k, v, scale, window, rows)
    return gate_merge(q[rows], gate_w, o_sp, lse_sp, o_w)


def tile_block_scores(T, block):
    """Block-level importance per query tile from the tile-token scores:
    M[t, c] = max over the keys of block c of T[t, j] (-inf when none is
    visible).  Block-level selection at the token budget of HySparse2 picks
    the top (budget / block) blocks of these rows ([deming] section 03:
    token- vs block-level selection at the same 1024 + 128 budget)."""
    T = np.asarray(T, dtype=np.float64)
    nt, Lk = T.shape
    nblk = (Lk + block - 1) // block
    pad = np.full((nt, nblk * block), NEG_INF)
    pad[:, :Lk] = T
    return pad.reshape(nt, nblk, block).max(axis=2)


def expand_blocks(sel_blocks, block, Lk):
    """Token positions of selected blocks (ascending, -1 padded): each block c
    contributes [c*block, min(Lk, (c+1)*block))."""
    sel_blocks = np.asarray(sel_blocks)
    out = np.full((sel_blocks.shape[0], sel_blocks.shape[1] * block), -1, dtype=np.int64)
    for r in range(sel_blocks.shape[0]):
        toks = [j for c in sel_blocks[r] if c >= 0 for j in range(c * block, min(Lk, (c + 1) * block))]
        out[r, :len(toks)] = toks
    return out
