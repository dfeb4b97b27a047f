"""Pins of the backward-pass oracle (oracle/hysparse_bwd.py).

Every gradient is checked element by element against central finite
differences of the forward definitions of oracle/hysparse.py (pinned on their
own), with the loss sum(dO * O) for random upstream gradients dO and the
selection held fixed.  The step h = 1e-5 in float64 leaves an error of order
h^2 * |third derivative| + eps / h, about 1e-9 here; the bound is 1e-6.
Reductions: an empty selection leaves only the window branch, and selecting
every block with a saturated gate gives the full layer's causal gradient.
"""
import numpy as np
import pytest

from oracle import hysparse as hs
from oracle import hysparse_bwd as hb

H = 1e-5
TOL = 1e-6


def _fd(f, x):
    """Central differences of the scalar f() with respect to every element of x (modified in place)."""
    g = np.zeros_like(x)
    it = np.nditer(x, flags=["multi_index"])
    for _ in it:
        ix = it.multi_index
        x0 = x[ix]
        x[ix] = x0 + H
        fp = f()
        x[ix] = x0 - H
        fm = f()
        x[ix] = x0
        g[ix] = (fp - fm) / (2 * H)
    return g


def _rand(seed, *shape, s=1.0):
    return s * np.random.default_rng(seed).standard_normal(shape)


@pytest.mark.parametrize("L,Hq,Hkv,D", [(19, 4, 2, 6), (24, 3, 1, 5)])
def test_full_attention_bwd_finite_differences(L, Hq, Hkv, D):
    q, k, v = _rand(1, L, Hq, D), _rand(2, L, Hkv, D), _rand(3, L, Hkv, D)
    do = _rand(4, L, Hq, D)
    scale = 0.4
    dq, dk, dv = hb.full_attention_bwd(q, k, v, scale, do)
    loss = lambda: float((do * hs.full_attention(q, k, v, scale)[0]).sum())
    for x, g in ((q, dq), (k, dk), (v, dv)):
        np.testing.assert_allclose(g, _fd(loss, x), rtol=0, atol=TOL)


def _layer_case(seed, L=40, Hq=4, Hkv=2, D=5, block=8, kb=2, window=6):
    q, k, v = _rand(seed, L, Hq, D), _rand(seed + 1, L, Hkv, D), _rand(seed + 2, L, Hkv, D)
    kw, vw = _rand(seed + 3, L, Hkv, D), _rand(seed + 4, L, Hkv, D)
    gw = _rand(seed + 5, Hq, D, s=0.5)
    do = _rand(seed + 6, L, Hq, D)
    sel, _ = hs.topk_rows(hs.block_scores(q, k, 0.45, block), kb)
    return q, k, v, kw, vw, gw, do, sel, block, window


def test_sparse_layer_bwd_finite_differences():
    q, k, v, kw, vw, gw, do, sel, block, window = _layer_case(10)
    scale = 0.45
    # rows whose selected blocks are all in the future have an empty sparse set
    # and take the window branch alone: both cases occur here
    r = hb.sparse_layer_bwd(q, k, v, kw, vw, gw, scale, sel, block, window, do)

    def loss():
        o_sp, lse_sp = hs.sparse_block_attention(q, k, v, scale, sel, block)
        o_w, _ = hs.window_attention(q, kw, vw, scale, window)
        return float((do * hs.gate_merge(q, gw, o_sp, lse_sp, o_w)).sum())
    for name, x in (("dq", q), ("dk", k), ("dv", v), ("dkw", kw), ("dvw", vw), ("dgate_w", gw)):
        np.testing.assert_allclose(r[name], _fd(loss, x), rtol=0, atol=TOL, err_msg=name)


def test_sparse_layer_bwd_per_group_sets_finite_differences():
    q, k, v, kw, vw, gw, do, _, block, window = _layer_case(20)
    scale = 0.45
    Mg = hs.block_scores_per_group(q, k, scale, block)
    sel_g = np.stack([hs.topk_rows(Mg[g], 2)[0] for g in range(k.shape[1])])
    r = hb.sparse_layer_bwd(q, k, v, kw, vw, gw, scale, None, block, window, do, sel_groups=sel_g)

    def loss():
        o_sp, lse_sp = hs.sparse_block_attention_grouped(q, k, v, scale, sel_g, block)
        o_w, _ = hs.window_attention(q, kw, vw, scale, window)
        return float((do * hs.gate_merge(q, gw, o_sp, lse_sp, o_w)).sum())
    for name, x in (("dq", q), ("dk", k), ("dv", v), ("dgate_w", gw)):
        np.testing.assert_allclose(r[name], _fd(loss, x), rtol=0, atol=TOL, err_msg=name)


def test_hysparse_block_bwd_finite_differences():
    L, Hq, Hkv, D, block, kb, window, scale = 33, 4, 2, 4, 8, 2, 5, 0.5
    ql = [_rand(30 + l, L, Hq, D) for l in range(3)]
    k, v = _rand(40, L, Hkv, D), _rand(41, L, Hkv, D)
    kw = [_rand(42 + l, L, Hkv, D) for l in range(2)]
    vw = [_rand(44 + l, L, Hkv, D) for l in range(2)]
    gw = [_rand(46 + l, Hq, D, s=0.5) for l in range(2)]
    do_full = _rand(50, L, Hq, D)
    do_l = [_rand(51 + l, L, Hq, D) for l in range(2)]
    r = hb.hysparse_block_bwd(ql, k, v, kw, vw, gw, scale, block, kb, window, do_full, do_l)
    sel = r["sel"]

    def loss():
        # the forward block with the selection held at the unperturbed one
        tot = float((do_full * hs.full_attention(ql[0], k, v, scale)[0]).sum())
        for l in range(2):
            o_sp, lse_sp = hs.sparse_block_attention(ql[l + 1], k, v, scale, sel, block)
            o_w, _ = hs.window_attention(ql[l + 1], kw[l], vw[l], scale, window)
            tot += float((do_l[l] * hs.gate_merge(ql[l + 1], gw[l], o_sp, lse_sp, o_w)).sum())
        return tot
    np.testing.assert_allclose(r["dk"], _fd(loss, k), rtol=0, atol=TOL)
    np.testing.assert_allclose(r["dv"], _fd(loss, v), rtol=0, atol=TOL)
    for l in range(3):
        np.testing.assert_allclose(r["dq"][l], _fd(loss, ql[l]), rtol=0, atol=TOL)
    np.testing.assert_allclose(r["dkw"][1], _fd(loss, kw[1]), rtol=0, atol=TOL)
    np.testing.assert_allclose(r["dgate_w"][0], _fd(loss, gw[0]), rtol=0, atol=TOL)


def test_empty_selection_is_the_window_branch_gradient():
    q, k, v, kw, vw, gw, do, sel, block, window = _layer_case(60)
    none = np.full_like(sel, -1)
    r = hb.sparse_layer_bwd(q, k, v, kw, vw, gw, 0.45, none, block, window, do)
    dq_w, dkw, dvw, _, _ = hb.masked_attention_bwd(q, kw, vw, 0.45, hb.window_allowed(40, 40, window), do)
    assert not r["dk"].any() and not r["dv"].any() and not r["dgate_w"].any()
    np.testing.assert_allclose(r["dq"], dq_w, rtol=0, atol=1e-12)
    np.testing.assert_allclose(r["dkw"], dkw, rtol=0, atol=1e-12)
    np.testing.assert_allclose(r["dvw"], dvw, rtol=0, atol=1e-12)


def test_all_blocks_and_saturated_gate_is_the_full_gradient():
    q, k, v, kw, vw, gw, do, sel, block, window = _layer_case(70)
    L = q.shape[0]
    every = np.tile(np.arange((L + block - 1) // block), (L, 1))
    q[:, :, 0] = 1.0
    w = np.zeros_like(gw)
    w[:, 0] = 40.0                       # g = sigmoid(40): 1 to 4e-18
    r = hb.sparse_layer_bwd(q, k, v, kw, vw, w, 0.45, every, block, window, do)
    dq, dk, dv = hb.full_attention_bwd(q, k, v, 0.45, do)
    np.testing.assert_allclose(r["dk"], dk, rtol=0, atol=1e-12)
    np.testing.assert_allclose(r["dv"], dv, rtol=0, atol=1e-12)
    np.testing.assert_allclose(r["dq"], dq, rtol=0, atol=1e-12)
    assert np.abs(r["dkw"]).max() < 1e-12 and np.abs(r["dgate_w"]).max() < 1e-12


def test_row_subsets_give_the_same_rows_and_last_keys():
    # dq of a row subset equals the full dq at those rows; the rows from the
    # first of the last keys on carry every contribution to those keys
    q, k, v, kw, vw, gw, do, sel, block, window = _layer_case(80, L=70)
    L = q.shape[0]
    full = hb.sparse_layer_bwd(q, k, v, kw, vw, gw, 0.45, sel, block, window, do)
    rows = np.arange(L - 20, L)
    part = hb.sparse_layer_bwd(q, k, v, kw, vw, gw, 0.45, sel[rows], block, window, do, rows=rows)
    np.testing.assert_allclose(part["dq"], full["dq"][rows], rtol=0, atol=1e-12)
    for name in ("dk", "dv", "dkw", "dvw"):
        np.testing.assert_allclose(part[name][L - 20:], full[name][L - 20:], rtol=0, atol=1e-12, err_msg=name)
    dq, dk, dv = hb.full_attention_bwd(q, k, v, 0.45, do)
    pq, pk, pv = hb.full_attention_bwd(q, k, v, 0.45, do, rows=rows)
    np.testing.assert_allclose(pq, dq[rows], rtol=0, atol=1e-12)
    np.testing.assert_allclose(pk[L - 20:], dk[L - 20:], rtol=0, atol=1e-12)
    np.testing.assert_allclose(pv[L - 20:], dv[L - 20:], rtol=0, atol=1e-12)


def test_sparse_layer_bwd_with_gate_bias_finite_differences():
    q, k, v, kw, vw, gw, do, sel, block, window = _layer_case(90)
    gb = _rand(96, q.shape[1], s=0.7)
    scale = 0.45
    r = hb.sparse_layer_bwd(q, k, v, kw, vw, gw, scale, sel, block, window, do, gate_b=gb)

    def loss():
        o_sp, lse_sp = hs.sparse_block_attention(q, k, v, scale, sel, block)
        o_w, _ = hs.window_attention(q, kw, vw, scale, window)
        return float((do * hs.gate_merge(q, gw, o_sp, lse_sp, o_w, gate_b=gb)).sum())
    for name, x in (("dgate_b", gb), ("dq", q), ("dgate_w", gw)):
        np.testing.assert_allclose(r[name], _fd(loss, x), rtol=0, atol=TOL, err_msg=name)


def test_gate_bias_saturates_the_gate():
    # a bias of +-60 gives g = 1 (sparse branch where it exists) or g = 0 (window branch)
    q, k, v, kw, vw, gw, do, sel, block, window = _layer_case(91)
    o_sp, lse_sp = hs.sparse_block_attention(q, k, v, 0.45, sel, block)
    o_w, _ = hs.window_attention(q, kw, vw, 0.45, window)
    live = np.isfinite(lse_sp.T)
    b = np.full(q.shape[1], 60.0)
    np.testing.assert_allclose(hs.gate_merge(q, 0 * gw, o_sp, lse_sp, o_w, gate_b=b)[live], o_sp[live], rtol=0, atol=1e-12)
    np.testing.assert_allclose(hs.gate_merge(q, 0 * gw, o_sp, lse_sp, o_w, gate_b=-b), o_w, rtol=0, atol=1e-12)
