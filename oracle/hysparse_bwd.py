"""Gradients of the HySparse hybrid block, in float64 (backward pass).

TEST INFRASTRUCTURE ONLY: imported by tests/, the package's smoke check and
the bench's CPU-baseline leg, never by the HIP path.

The pages say the hybrid structure is trained directly ([QbitAI] opening
summary; [deming] section 06) but print no backward pass, so the functions
here are the plain derivatives of the forward definitions in
oracle/hysparse.py with the selection held fixed: top-k is piecewise
constant in the scores, so it passes no gradient, and the sparse layers'
index sets are inputs of the backward exactly as they are of the forward.

For one attention branch with visible set J(i) per query row and head,
  P = softmax_J(S),  S = scale * q k^T,  O = P v,
the derivatives of a loss with upstream gradient dO are
  dV   = P^T dO
  dP   = dO v^T
  dS   = P * (dP - rowsum(dO * O))
  dQ   = scale * dS k,   dK = scale * dS^T q,
with the sums over the G query heads of a KV head collected in that head's
dK, dV.  The sparse layer's gate o = g O_sp + (1 - g) O_w,
g = sigmoid(<q, w_h> + b_h), adds
  dO_sp = g dO,  dO_w = (1 - g) dO,  dz = g (1 - g) <dO, O_sp - O_w>,
  dq += dz w_h,  dw_h = sum over rows of dz q,  db_h = sum over rows of dz,
and a row whose selected set is empty has o = O_w (no gate term, no sparse
branch).  The shared K/V receive the full layer's gradient plus every
sparse layer's sparse-branch gradient; each layer's own window K/V only its
window branch's.  A key's gradient collects every query row that sees it;
the functions can evaluate a subset of the rows, which gives dQ of those rows
exactly and the key gradients of keys that no other row sees (the last keys
of a long sequence).  The functions are pinned by central finite
differences of the forward definitions (tests/test_oracle_bwd.py).
"""
from __future__ import annotations

import numpy as np

from .hysparse import NEG_INF, block_scores, logits, topk_rows


def _row_ids(rows, L):
    return np.arange(L) if rows is None else np.asarray(rows, dtype=np.int64)


def _causal(L: int, Lk: int, rows=None) -> np.ndarray:
    i = _row_ids(rows, L)[:, None]
    j = np.arange(Lk)[None, :]
    return j <= i


def block_allowed(sel, block: int, L: int, Lk: int, rows=None) -> np.ndarray:
    """Visible set of the block-sparse branch: j <= i and j // block in sel[r]
    for the r-th of the query rows `rows` (all L rows by default)."""
    ids = _row_ids(rows, L)
    allowed = np.zeros((len(ids), Lk), dtype=bool)
    for r in range(len(ids)):
        for c in np.asarray(sel[r]):
            if c >= 0:
                allowed[r, c * block:(c + 1) * block] = True
    return allowed & _causal(L, Lk, rows)


def window_allowed(L: int, Lk: int, window: int, rows=None) -> np.ndarray:
    """Visible set of the window branch: i - window < j <= i."""
    i = _row_ids(rows, L)[:, None]
    j = np.arange(Lk)[None, :]
    return (j <= i) & (j > i - window)


def masked_attention_bwd(q, k, v, scale, allowed, do):
    """Backward of softmax attention over a visible set.

    q [L, Hq, D]; k, v [Lk, Hkv, D]; allowed [L, Lk] (one set for every head)
    or [Hq, L, Lk]; do [L, Hq, D].  Returns dq [L, Hq, D], dk, dv [Lk, Hkv, D],
    and the forward's O [L, Hq, D] and LSE [Hq, L] (a row with nothing visible
    has O = 0, LSE = -inf and passes no gradient).
    """
    L, Hq, D = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    S = logits(q, k, scale, G)
    mask = np.broadcast_to(allowed, S.shape)
    S = np.where(mask, S, NEG_INF)
    dq = np.zeros_like(q)
    dk = np.zeros(k.shape, dtype=np.float64)
    dv = np.zeros(v.shape, dtype=np.float64)
    O = np.zeros((L, Hq, D), dtype=np.float64)
    lse = np.full((Hq, L), NEG_INF)
    for h in range(Hq):
        g = h // G
        m = S[h].max(axis=1)
        live = np.isfinite(m)
        m0 = np.where(live, m, 0.0)
        E = np.exp(S[h] - m0[:, None])
        den = E.sum(axis=1)
        P = np.where(live[:, None], E / np.where(live, den, 1.0)[:, None], 0.0)
        O[:, h] = P @ v[:, g]
        lse[h] = np.where(live, m0 + np.log(np.where(live, den, 1.0)), NEG_INF)
        dv[:, g] += P.T @ do[:, h]
        dP = do[:, h] @ v[:, g].T
        Dd = (do[:, h] * O[:, h]).sum(axis=1)
        dS = P * (dP - Dd[:, None])
        dq[:, h] = scale * (dS @ k[:, g])
        dk[:, g] += scale * (dS.T @ q[:, h])
    return dq, dk, dv, O, lse


def full_attention_bwd(q, k, v, scale, do, rows=None):
    """Backward of the full layer's causal attention.

    With `rows`, only those query rows are evaluated: dq is theirs, and dk, dv
    hold their rows' contributions, which is the whole gradient of every key
    that only those rows see (for example the last keys when `rows` are the
    rows from the first of them to the end)."""
    ids = _row_ids(rows, q.shape[0])
    dq, dk, dv, _, _ = masked_attention_bwd(q[ids], k, v, scale, _causal(q.shape[0], k.shape[0], rows), do[ids])
    return dq, dk, dv


def sparse_layer_bwd(q, k, v, kw, vw, gate_w, scale, sel, block, window, do, sel_groups=None, rows=None,
                     gate_b=None):
    """Backward of one HySparse sparse layer (block-sparse branch over the
    shared k/v, window branch over the layer's kw/vw, sigmoid gate).

    sel [R, kb]: the block ids of each evaluated query row (one set for all
    heads), or sel_groups [Hkv, R, kb]: one set per KV group (head h uses
    h // G).  The rows are all L rows, or those in `rows` (then dq is theirs
    and the key gradients and dgate_w hold their contributions only, as in
    full_attention_bwd).  gate_b: the gate's optional per-head bias.  Returns
    dict(dq, dk, dv, dkw, dvw, dgate_w, dgate_b) with dk, dv the contribution
    to the shared cache and dgate_b the row sum of dz per head.
    """
    L, Hq, D = q.shape
    Lk = k.shape[0]
    ids = _row_ids(rows, L)
    if sel_groups is None:
        allowed_sp = block_allowed(sel, block, L, Lk, rows)
    else:
        Hkv = k.shape[1]
        G = Hq // Hkv
        allowed_sp = np.stack([block_allowed(sel_groups[h // G], block, L, Lk, rows) for h in range(Hq)])
    allowed_w = window_allowed(L, kw.shape[0], window, rows)
    q, do = q[ids], do[ids]
    # forward of the two branches (their O and LSE are what the gate needs)
    zero = np.zeros_like(do)
    _, _, _, o_sp, lse_sp = masked_attention_bwd(q, k, v, scale, allowed_sp, zero)
    _, _, _, o_w, _ = masked_attention_bwd(q, kw, vw, scale, allowed_w, zero)
    z = np.einsum("lhd,hd->lh", q, gate_w)
    if gate_b is not None:
        z = z + np.asarray(gate_b)[None, :]
    g = 1.0 / (1.0 + np.exp(-z))
    on = np.isfinite(lse_sp.T)                                   # [L, Hq]: the sparse branch exists
    g_eff = np.where(on, g, 0.0)
    dz = np.where(on, g * (1.0 - g) * (do * (o_sp - o_w)).sum(axis=2), 0.0)
    dq_sp, dk, dv, _, _ = masked_attention_bwd(q, k, v, scale, allowed_sp, g_eff[:, :, None] * do)
    dq_w, dkw, dvw, _, _ = masked_attention_bwd(q, kw, vw, scale, allowed_w, (1.0 - g_eff)[:, :, None] * do)
    dq = dq_sp + dq_w + dz[:, :, None] * gate_w[None, :, :]
    dgate_w = np.einsum("lh,lhd->hd", dz, q)
    return dict(dq=dq, dk=dk, dv=dv, dkw=dkw, dvw=dvw, dgate_w=dgate_w, dgate_b=dz.sum(axis=0))


def hysparse_block_bwd(q_layers, k, v, kw_layers, vw_layers, gate_layers, scale, block, topk, window,
                       do_full, do_layers):
    """Backward of one HySparse hybrid block (one sequence).

    The selection is the forward's (block scores of the full layer, top-k per
    row) and is returned with the gradients.  dk, dv sum the full layer's
    gradient and every sparse layer's sparse-branch gradient (the shared
    cache); dq[l], dkw[l], dvw[l], dgate_w[l] are per layer (l = 0 the full
    layer for dq; window and gate lists start at the first sparse layer).
    """
    q0 = q_layers[0]
    sel, _ = topk_rows(block_scores(q0, k, scale, block), topk)
    dq0, dk, dv = full_attention_bwd(q0, k, v, scale, do_full)
    dq, dkw, dvw, dgw = [dq0], [], [], []
    for l in range(1, len(q_layers)):
        r = sparse_layer_bwd(q_layers[l], k, v, kw_layers[l - 1], vw_layers[l - 1], gate_layers[l - 1], scale,
                             sel, block, window, do_layers[l - 1])
        dk = dk + r["dk"]
        dv = dv + r["dv"]
        dq.append(r["dq"])
        dkw.append(r["dkw"])
        dvw.append(r["dvw"])
        dgw.append(r["dgate_w"])
    return dict(sel=sel, dq=dq, dk=dk, dv=dv, dkw=dkw, dvw=dvw, dgate_w=dgw)
