"""HySparse (block-level) decode step with ring window caches.

TEST INFRASTRUCTURE ONLY (see the package header).

The HySparse pages describe the hybrid block for prefill; decoding the same
structure needs, per step and sequence (one new query at position n-1, the
shared cache already holding keys [0, n)):

  * the full layer: exact attention of the new query over keys [0, n) and the
    block importance of that one query, M[c] = max over query heads and over
    the keys of 64-token block c that are < n (QbitAI HySparse article, method
    section; TechWalker write-up: the full layer's kernel emits block-level
    maxima; -inf for blocks with no key below n);
  * the top-k blocks of M (the same selection rule as prefill);
  * each sparse layer: the block-sparse branch over the selected blocks of the
    shared cache, the sliding-window branch over the layer's own window K/V
    (the last W = 128 tokens, kept independently: TechWalker write-up), and
    the sigmoid gate that fuses them (QbitAI article).

Readings (the pages are silent on decode mechanics):
  * a sparse layer's window cache is a ring of W slots: token t lives in slot
    t mod W.  Before the step the ring holds the tokens [n-1-W, n-2] that
    exist; the step writes the new token's window K/V (an input here: the
    layer's own projection is outside the attention path) into slot
    (n-1) mod W, and the window branch then covers tokens [max(0, n-W), n-1];
  * the block-score row is ceil(Nmax / 64) wide for a cache of capacity Nmax,
    so sequences of different lengths share one layout.
A decode step is then exactly the prefill block evaluated at row n-1 (pinned
in tests/test_oracle_hysparse_decode.py against the prefill functions).
"""
import numpy as np

from .hysparse import NEG_INF, attend, decode_full, gate_merge, logits, topk_select


def ring_slot(t: int, W: int) -> int:
    """Slot of token t in a W-slot ring."""
    return int(t) % int(W)


def ring_append(ring_k, ring_v, k_new, v_new, n):
    """Copies of one sequence's ring [W, Hkv, D] with token n-1 written into its slot."""
    rk = np.array(ring_k, dtype=np.float64, copy=True)
    rv = np.array(ring_v, dtype=np.float64, copy=True)
    s = ring_slot(n - 1, rk.shape[0])
    rk[s] = k_new
    rv[s] = v_new
    return rk, rv


def ring_window(ring_k, ring_v, n):
    """The window tokens [max(0, n-W), n-1] of a ring, in position order.

    Returns (k [m, Hkv, D], v [m, Hkv, D], positions [m]).
    """
    W = ring_k.shape[0]
    pos = np.arange(max(0, n - W), n, dtype=np.int64)
    slots = pos % W
    return ring_k[slots], ring_v[slots], pos


def block_scores_decode(token_scores, n, block, nblk):
    """M[c] = max of the token scores over the keys of block c below n; -inf if none."""
    s = np.full(nblk * block, NEG_INF)
    s[:n] = np.asarray(token_scores, dtype=np.float64)[:n]
    return s.reshape(nblk, block).max(axis=1)


def sparse_blocks_decode(qd, kc, vc, scale, n, sel, block):
    """Block-sparse branch at decode: J = {j < n : j // block in sel}.

    qd [Hq, D]; kc, vc [N, Hkv, D].  Returns O [Hq, D], LSE [Hq] (-inf, O = 0 when J is empty).
    """
    Hq = qd.shape[0]
    G = Hq // kc.shape[1]
    allowed = np.zeros(n, dtype=bool)
    for c in np.asarray(sel):
        if c >= 0:
            allowed[c * block:min(n, (c + 1) * block)] = True
    S = logits(qd[None], kc[:n], scale, G)
    S[:, 0, ~allowed] = NEG_INF
    O, lse = attend(S, vc[:n], G)
    return O[0], lse[:, 0]


def window_decode(qd, kw, vw, scale):
    """Window branch at decode: attention over all given window keys kw, vw [m, Hkv, D]."""
    Hq = qd.shape[0]
    G = Hq // kw.shape[1]
    S = logits(qd[None], kw, scale, G)
    O, _ = attend(S, vw, G)
    return O[0]


def hysparse_decode_step(q_full, kc, vc, scale, n, nmax, q_sparse, k_rings, v_rings, k_new, v_new,
                         gate_ws, block, topk):
    """One HySparse decode step for one sequence of valid length n (cache capacity nmax).

    q_full [Hq, D]; kc, vc [nmax, Hkv, D]; per sparse layer l: q_sparse[l] [Hq, D],
    k_rings[l], v_rings[l] [W, Hkv, D] (before the append), k_new[l], v_new[l]
    [Hkv, D], gate_ws[l] [Hq, D].  Returns the full layer's output and scores,
    the selection, each sparse layer's output and the rings after the append.
    """
    o_full, lse, s = decode_full(q_full, kc, vc, scale, n)
    nblk = (int(nmax) + block - 1) // block
    M = block_scores_decode(s, n, block, nblk)
    sel, cnt = topk_select(M, topk)
    outs, rings = [], []
    for l in range(len(q_sparse)):
        ql = np.asarray(q_sparse[l], dtype=np.float64)
        rk, rv = ring_append(k_rings[l], v_rings[l], k_new[l], v_new[l], n)
        kw, vw, _ = ring_window(rk, rv, n)
        o_sp, lse_sp = sparse_blocks_decode(ql, kc, vc, scale, n, sel, block)
        o_w = window_decode(ql, kw, vw, scale)
        o = gate_merge(ql[None], np.asarray(gate_ws[l], dtype=np.float64), o_sp[None], lse_sp[:, None], o_w[None])[0]
        outs.append(o)
        rings.append((rk, rv))
    return dict(o_full=o_full, lse=lse, token_scores=s, block_scores=M, sel=sel, count=cnt,
                o_layers=outs, rings=rings)
