"""Pins of the fp64 CPU oracle against things other than itself.

Brute force (pure-Python loops), torch's CPU float64 SDPA, closed forms,
invariants, special cases and the hand-derived golden files.  Each check is
chosen so that a plausible slip in the oracle (a dropped scale, a wrong head
mapping, an off-by-one mask, a reversed tie rule) fails at least one of them.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from tests import brute_force as bf

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _tolist(a):
    return np.asarray(a).tolist()


def _case(L=37, Hq=4, Hkv=2, D=8, seed=0):
    q = _rand((L, Hq, D), seed)
    k = _rand((L, Hkv, D), seed + 1)
    v = _rand((L, Hkv, D), seed + 2)
    return q, k, v, 1.0 / math.sqrt(D)


def _f(x):
    return float("-inf") if x == "-inf" else (float("nan") if x == "nan" else float(x))


# ----------------------------------------------------------------------------
# golden, hand-derived values
# ----------------------------------------------------------------------------

def test_golden_softmax_closed_form():
    g = json.load(open(os.path.join(GOLD, "softmax_closed_form.json")))
    q = np.array(g["q"]).reshape(3, 1, 1)
    k = np.array(g["k"]).reshape(3, 1, 1)
    v = np.array(g["v"]).reshape(3, 1, 1)
    O, lse = oracle.full_attention(q, k, v, g["scale"])
    np.testing.assert_allclose(O[:, 0, 0], g["o"], rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse[0], g["lse"], rtol=0, atol=1e-14)
    M = oracle.block_scores(q, k, g["scale"], g["block"])
    exp = np.array([[_f(x) for x in row] for row in g["block_scores"]])
    assert np.array_equal(np.isinf(M), np.isinf(exp))
    np.testing.assert_allclose(M[np.isfinite(exp)], exp[np.isfinite(exp)], atol=1e-14)
    idx, cnt = oracle.topk_select(M[2], 1)
    assert idx.tolist() == g["top1_row2"] and cnt == 1


def test_golden_topk_ties():
    g = json.load(open(os.path.join(GOLD, "topk_ties.json")))
    x = np.array([_f(s) for s in g["scores"]])
    for c in g["cases"]:
        idx, cnt = oracle.topk_select(x, c["k"])
        assert idx.tolist() == c["idx"], c
        assert cnt == c["count"]


def test_golden_gate_closed_form():
    g = json.load(open(os.path.join(GOLD, "gate_closed_form.json")))
    q = np.array(g["q"]).reshape(1, 1, 2)
    w = np.array(g["w"]).reshape(1, 2)
    o_sp = np.array(g["o_sp"]).reshape(1, 1, 2)
    o_w = np.array(g["o_w"]).reshape(1, 1, 2)
    out = oracle.gate_merge(q, w, o_sp, np.zeros((1, 1)), o_w)
    np.testing.assert_allclose(out[0, 0], g["o"], atol=1e-14)
    out = oracle.gate_merge(q, w, o_sp, np.full((1, 1), -np.inf), o_w)
    np.testing.assert_allclose(out[0, 0], g["o_empty"], atol=0)


# ----------------------------------------------------------------------------
# a1 full attention
# ----------------------------------------------------------------------------

def test_full_attention_brute_force():
    q, k, v, sc = _case(L=23, Hq=4, Hkv=2, D=6)
    O, lse = oracle.full_attention(q, k, v, sc)
    Ob, lseb = bf.attention(_tolist(q), _tolist(k), _tolist(v), sc, lambda i, j: j <= i)
    np.testing.assert_allclose(O, np.array(Ob), rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, np.array(lseb), rtol=0, atol=1e-12)


@pytest.mark.parametrize("Hq,Hkv", [(8, 1), (4, 4), (8, 2)])
def test_full_attention_vs_torch_sdpa(Hq, Hkv):
    L, D = 300, 16
    q, k, v, sc = _case(L=L, Hq=Hq, Hkv=Hkv, D=D, seed=5)
    O, _ = oracle.full_attention(q, k, v, sc)
    G = Hq // Hkv
    tq = torch.from_numpy(q).permute(1, 0, 2)[None]
    tk = torch.from_numpy(k).permute(1, 0, 2).repeat_interleave(G, dim=0)[None]
    tv = torch.from_numpy(v).permute(1, 0, 2).repeat_interleave(G, dim=0)[None]
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=True, scale=sc)
    np.testing.assert_allclose(O, ref[0].permute(1, 0, 2).numpy(), rtol=0, atol=1e-12)


def test_full_attention_invariants():
    q, k, v, sc = _case(L=64, Hq=4, Hkv=1, D=8, seed=3)
    # V == 1 everywhere -> O == 1: the softmax weights of every row sum to 1.
    O1, _ = oracle.full_attention(q, k, np.ones_like(v), sc)
    np.testing.assert_allclose(O1, 1.0, atol=1e-13)
    # Row 0 sees only key 0.
    O, _ = oracle.full_attention(q, k, v, sc)
    for h in range(4):
        np.testing.assert_allclose(O[0, h], v[0, 0], atol=1e-14)
    # Each output coordinate lies inside the range of the visible V rows.
    for i in range(64):
        lo, hi = v[:i + 1, 0].min(axis=0), v[:i + 1, 0].max(axis=0)
        assert np.all(O[i] >= lo - 1e-12) and np.all(O[i] <= hi + 1e-12)
    # Constant keys -> uniform weights -> prefix mean of V.
    kc = np.broadcast_to(k[:1], k.shape).copy()
    Oc, lsec = oracle.full_attention(q, kc, v, sc)
    pm = np.cumsum(v[:, 0], axis=0) / np.arange(1, 65)[:, None]
    for h in range(4):
        np.testing.assert_allclose(Oc[:, h], pm, atol=1e-12)
    # With constant keys the LSE is the common logit plus ln(i+1).
    s0 = sc * (q[:, 0] @ k[0, 0])
    np.testing.assert_allclose(lsec[0], s0 + np.log(np.arange(1, 65)), atol=1e-12)


def test_split_merge_rule():
    """LSE merge of two disjoint key chunks equals the unchunked softmax.

    This is the combine rule a split-K kernel uses:
      m = max(m1, m2);  l = l1 e^{m1-m} + l2 e^{m2-m};  O = (O1 l1 e^{m1-m} + O2 l2 e^{m2-m}) / l
    written here with LSEs: w_c = exp(lse_c - lse), lse = ln(e^{lse1} + e^{lse2}).
    """
    q, k, v, sc = _case(L=50, Hq=2, Hkv=1, D=8, seed=9)
    i = 49
    S = oracle.logits(q[[i]], k, sc, 2)
    O, lse = oracle.attend(S, v, 2)
    S1, S2 = S.copy(), S.copy()
    S1[:, :, 20:] = -np.inf
    S2[:, :, :20] = -np.inf
    O1, l1 = oracle.attend(S1, v, 2)
    O2, l2 = oracle.attend(S2, v, 2)
    lm = np.logaddexp(l1, l2)
    Om = np.exp(l1 - lm).T[:, :, None] * O1 + np.exp(l2 - lm).T[:, :, None] * O2
    np.testing.assert_allclose(Om, O, atol=1e-13)
    np.testing.assert_allclose(lm, lse, atol=1e-13)


# ----------------------------------------------------------------------------
# a2 importance scores
# ----------------------------------------------------------------------------

def test_block_scores_brute_force():
    q, k, v, sc = _case(L=45, Hq=4, Hkv=2, D=5, seed=11)
    M = oracle.block_scores(q, k, sc, 8)
    Mb = np.array(bf.block_scores(_tolist(q), _tolist(k), sc, 8))
    assert np.array_equal(np.isinf(M), np.isinf(Mb))
    np.testing.assert_allclose(M[np.isfinite(M)], Mb[np.isfinite(Mb)], atol=1e-12)


def test_block_scores_row_max_and_ties():
    q, k, v, sc = _case(L=128, Hq=4, Hkv=2, D=8, seed=12)
    M = oracle.block_scores(q, k, sc, 16)
    # max over blocks = the row max of the logits over heads and visible keys
    S = oracle.logits(q, k, sc, 2)
    S[:, np.triu(np.ones((128, 128), bool), 1)] = -np.inf
    np.testing.assert_allclose(M.max(axis=1), S.max(axis=(0, 2)), atol=1e-13)
    # future blocks are -inf
    for i in range(128):
        assert np.all(np.isneginf(M[i, i // 16 + 1:]))
        assert np.all(np.isfinite(M[i, :i // 16 + 1]))
    # two identical key blocks give identical scores
    k2 = k.copy()
    k2[32:48] = k2[16:32]
    M2 = oracle.block_scores(q, k2, sc, 16)
    assert np.array_equal(M2[60:, 1], M2[60:, 2])


def test_tile_token_scores_brute_force():
    q, k, v, sc = _case(L=29, Hq=4, Hkv=1, D=6, seed=13)
    T = oracle.tile_token_scores(q, k, sc, 8)
    Tb = np.array(bf.tile_token_scores(_tolist(q), _tolist(k), sc, 8))
    assert np.array_equal(np.isinf(T), np.isinf(Tb))
    np.testing.assert_allclose(T[np.isfinite(T)], Tb[np.isfinite(Tb)], atol=1e-12)


def test_tile_token_scores_tile1_is_decode_scores():
    q, k, v, sc = _case(L=40, Hq=4, Hkv=1, D=8, seed=14)
    T = oracle.tile_token_scores(q, k, sc, 1)
    for n in (1, 7, 40):
        _, _, s = oracle.decode_full(q[n - 1], k, v, sc, n)
        np.testing.assert_allclose(T[n - 1, :n], s, atol=1e-14)
        assert np.all(np.isneginf(T[n - 1, n:]))
    # a tile's row is the max over its rows' per-query token maxima
    T8 = oracle.tile_token_scores(q, k, sc, 8)
    np.testing.assert_allclose(T8[2], T[16:24].max(axis=0), atol=0)


# ----------------------------------------------------------------------------
# a3 top-k
# ----------------------------------------------------------------------------

def test_topk_vs_sorted_and_invariants():
    r = np.random.default_rng(21)
    for trial in range(200):
        n = int(r.integers(1, 80))
        x = np.round(r.standard_normal(n), 1)          # many ties
        x[r.random(n) < 0.1] = -np.inf
        k = int(r.integers(0, n + 3))
        idx, cnt = oracle.topk_select(x, k)
        exp, ecnt = bf.topk(x.tolist(), k)
        assert idx.tolist() == exp and cnt == ecnt
        chosen = set(idx[idx >= 0].tolist())
        rest = [c for c in range(n) if c not in chosen and np.isfinite(x[c])]
        if chosen and rest:
            assert min(x[list(chosen)]) >= max(x[rest])
        assert all(a < b for a, b in zip(idx[:cnt], idx[1:cnt]))


def test_topk_nan_and_neg_inf_never_chosen():
    x = np.array([np.nan, -np.inf, 0.5, np.nan, -np.inf])
    idx, cnt = oracle.topk_select(x, 4)
    assert idx.tolist() == [2, -1, -1, -1] and cnt == 1


def test_topk_lowest_index_wins_ties():
    x = np.zeros(10)
    idx, cnt = oracle.topk_select(x, 3)
    assert idx.tolist() == [0, 1, 2]
    x[7] = 1.0
    idx, _ = oracle.topk_select(x, 3)
    assert idx.tolist() == [0, 1, 7]


# ----------------------------------------------------------------------------
# a4 sparse branch
# ----------------------------------------------------------------------------

def test_sparse_block_all_blocks_is_full_attention():
    q, k, v, sc = _case(L=70, Hq=4, Hkv=2, D=8, seed=31)
    nblk = 9
    sel = np.tile(np.arange(nblk), (70, 1))
    O, lse = oracle.sparse_block_attention(q, k, v, sc, sel, 8)
    Of, lsef = oracle.full_attention(q, k, v, sc)
    np.testing.assert_allclose(O, Of, atol=1e-13)
    np.testing.assert_allclose(lse, lsef, atol=1e-13)


def test_sparse_block_brute_force_and_empty():
    q, k, v, sc = _case(L=40, Hq=4, Hkv=2, D=6, seed=32)
    r = np.random.default_rng(3)
    sel = np.full((40, 3), -1)
    for i in range(40):
        c = r.choice(5, size=int(r.integers(0, 4)), replace=False)
        sel[i, :len(c)] = np.sort(c)
    O, lse = oracle.sparse_block_attention(q, k, v, sc, sel, 8)
    allowed = {(i, j) for i in range(40) for j in range(40)
               if j <= i and (j // 8) in set(sel[i][sel[i] >= 0].tolist())}
    Ob, lseb = bf.attention(_tolist(q), _tolist(k), _tolist(v), sc, lambda i, j: (i, j) in allowed)
    for i in range(40):
        for h in range(4):
            if Ob[i][h] is None:
                assert np.isneginf(lse[h, i]) and np.all(O[i, h] == 0)
            else:
                np.testing.assert_allclose(O[i, h], Ob[i][h], atol=1e-12)
                assert abs(lse[h, i] - lseb[h][i]) < 1e-12


def test_sparse_token_special_cases():
    q, k, v, sc = _case(L=90, Hq=4, Hkv=1, D=8, seed=33)
    tile, W = 8, 16
    nt = 12
    # all tokens selected -> full attention
    sel_all = np.tile(np.arange(90), (nt, 1))
    O, _ = oracle.sparse_token_attention(q, k, v, sc, sel_all, tile, W)
    Of, _ = oracle.full_attention(q, k, v, sc)
    np.testing.assert_allclose(O, Of, atol=1e-13)
    # nothing selected (k = 0) -> pure window attention over the same K/V
    O0, _ = oracle.sparse_token_attention(q, k, v, sc, np.zeros((nt, 0), int), tile, W)
    Ow, _ = oracle.window_attention(q, k, v, sc, W)
    np.testing.assert_allclose(O0, Ow, atol=1e-13)
    # selection inside every query's window -> still window attention (no double counting)
    sel_in = np.array([[max(0, t * tile - 1)] for t in range(nt)])
    Oi, _ = oracle.sparse_token_attention(q, k, v, sc, sel_in, tile, W)
    np.testing.assert_allclose(Oi, Ow, atol=1e-13)


def test_sparse_token_brute_force():
    q, k, v, sc = _case(L=33, Hq=2, Hkv=1, D=4, seed=34)
    tile, W = 8, 4
    r = np.random.default_rng(5)
    sel = np.stack([np.sort(r.choice(33, 5, replace=False)) for _ in range(5)])
    O, _ = oracle.sparse_token_attention(q, k, v, sc, sel, tile, W)

    def vis(i, j):
        return j <= i and (j in set(sel[i // tile].tolist()) or j >= i - W + 1)
    Ob, _ = bf.attention(_tolist(q), _tolist(k), _tolist(v), sc, vis)
    np.testing.assert_allclose(O, np.array(Ob), atol=1e-12)


# ----------------------------------------------------------------------------
# a5 window + gate
# ----------------------------------------------------------------------------

def test_window_special_cases():
    q, k, v, sc = _case(L=50, Hq=4, Hkv=2, D=8, seed=41)
    Ow, _ = oracle.window_attention(q, k, v, sc, 50)
    Of, _ = oracle.full_attention(q, k, v, sc)
    np.testing.assert_allclose(Ow, Of, atol=1e-13)
    O1, _ = oracle.window_attention(q, k, v, sc, 1)
    for h in range(4):
        np.testing.assert_allclose(O1[:, h], v[:, h // 2], atol=1e-14)
    Ob, _ = bf.attention(_tolist(q), _tolist(k), _tolist(v), sc, lambda i, j: i - 7 <= j <= i)
    O7, _ = oracle.window_attention(q, k, v, sc, 8)
    np.testing.assert_allclose(O7, np.array(Ob), atol=1e-12)


def test_gate_special_cases():
    r = np.random.default_rng(42)
    q = r.standard_normal((5, 3, 4))
    o_sp = r.standard_normal((5, 3, 4))
    o_w = r.standard_normal((5, 3, 4))
    out = oracle.gate_merge(q, np.zeros((3, 4)), o_sp, np.zeros((3, 5)), o_w)
    np.testing.assert_allclose(out, 0.5 * (o_sp + o_w), atol=1e-15)
    w = r.standard_normal((3, 4))
    out = oracle.gate_merge(q, w, o_sp, np.zeros((3, 5)), o_w)
    for i in range(5):
        for h in range(3):
            g = bf.sigmoid(sum(q[i, h, d] * w[h, d] for d in range(4)))
            np.testing.assert_allclose(out[i, h], g * o_sp[i, h] + (1 - g) * o_w[i, h], atol=1e-14)


def test_block_k0_reproduces_window():
    """k = 0: the sparse set is empty, so the gated layer equals its window branch."""
    q, k, v, sc = _case(L=64, Hq=4, Hkv=1, D=8, seed=43)
    kw, vw = _rand((64, 1, 8), 44), _rand((64, 1, 8), 45)
    w = _rand((4, 8), 46) * 0.02
    res = oracle.hysparse_block([q, q], k, v, [kw], [vw], [w], sc, 16, 0, 16)
    Ow, _ = oracle.window_attention(q, kw, vw, sc, 16)
    np.testing.assert_allclose(res["o_layers"][0], Ow, atol=0)


# ----------------------------------------------------------------------------
# a6 decode
# ----------------------------------------------------------------------------

def test_decode_matches_prefill_rows():
    q, k, v, sc = _case(L=100, Hq=4, Hkv=1, D=8, seed=51)
    for n in (1, 37, 100):
        o, lse, s = oracle.decode_full(q[n - 1], k, v, sc, n)
        Of, lsef = oracle.full_attention(q, k, v, sc, rows=[n - 1])
        np.testing.assert_allclose(o, Of[0], atol=1e-13)
        np.testing.assert_allclose(lse, lsef[:, 0], atol=1e-13)
        sel, _ = oracle.topk_select(s, 10)
        osp, _ = oracle.decode_sparse(q[n - 1], k, v, sc, n, sel, 16)
        sel_tiles = np.full((100, 10), -1)
        sel_tiles[n - 1] = sel
        Ot, _ = oracle.sparse_token_attention(q, k, v, sc, sel_tiles, 1, 16, rows=[n - 1])
        np.testing.assert_allclose(osp, Ot[0], atol=1e-13)


def test_decode_k_large_is_full():
    q, k, v, sc = _case(L=60, Hq=4, Hkv=1, D=8, seed=52)
    res = oracle.decode_step(q[59], k, v, sc, 60, [q[10]], 100, 16)
    o, _, _ = oracle.decode_full(q[10], k, v, sc, 60)
    np.testing.assert_allclose(res["o_layers"][0], o, atol=1e-13)
    assert res["count"] == 60


# ----------------------------------------------------------------------------
# fp8 codec
# ----------------------------------------------------------------------------

def test_fp8_table_vs_torch():
    tab = oracle.fp8.decode_table()
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(tab), np.isnan(ref))
    np.testing.assert_array_equal(tab[~np.isnan(tab)], ref[~np.isnan(ref)])
    assert np.nanmax(tab) == 448.0 and np.isnan(tab[0x7F]) and np.isnan(tab[0xFF])
    assert tab[0x01] == 2.0 ** -9 and tab[0x08] == 2.0 ** -6


def test_fp8_exact_in_bf16():
    """Every finite e4m3 value is exactly representable in bf16."""
    tab = oracle.fp8.decode_table()
    fin = tab[np.isfinite(tab)]
    back = torch.from_numpy(fin).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(back, fin)


# ----------------------------------------------------------------------------
# O9 for HySparse2: the whole block evaluated for chosen query tiles
# ----------------------------------------------------------------------------

def test_hysparse2_block_brute_force_tiles_out_of_order():
    """Every field of hysparse2_block against pure-Python loops, for tiles
    requested out of order and a ragged last tile (L = 43, tile 8: tile 5 has
    three rows).  The brute force forms the tile-token scores, takes each
    tile's top-k with the lowest index winning ties, and attends each sparse
    layer over {selected tokens of the row's tile} U {the last W keys}, so a
    slip in the tile-to-row bookkeeping (rows out of the tiles' order, one
    tile's selection given to another, a window off by one) fails here."""
    q0, k, v, sc = _case(L=43, Hq=2, Hkv=1, D=4, seed=61)
    q1 = _rand((43, 2, 4), 62)
    q2 = _rand((43, 2, 4), 63)
    tile, topk, W = 8, 5, 4
    tiles = [4, 0, 5, 2]
    res = oracle.hysparse2_block([q0, q1, q2], k, v, sc, tile, topk, W, tiles=tiles)
    rows_ref = [i for t in tiles for i in range(t * tile, min(43, (t + 1) * tile))]
    assert res["rows"].tolist() == rows_ref
    T = bf.tile_token_scores(_tolist(q0), _tolist(k), sc, tile)
    for n, t in enumerate(tiles):
        np.testing.assert_allclose(res["scores"][n], np.array(T[t]), atol=1e-12)
        sel_t, cnt = bf.topk(T[t], topk)
        assert res["sel"][n].tolist() == sel_t and res["count"][n] == cnt
    Of, lse = bf.attention(_tolist(q0), _tolist(k), _tolist(v), sc, lambda i, j: j <= i)
    np.testing.assert_allclose(res["o_full"], np.array([Of[i] for i in rows_ref]), atol=1e-12)
    np.testing.assert_allclose(res["lse"], np.array([[lse[h][i] for i in rows_ref] for h in range(2)]), atol=1e-12)
    sel_of_tile = {t: set(c for c in bf.topk(T[t], topk)[0] if c >= 0) for t in tiles}
    for l, ql in enumerate((q1, q2)):
        Ob, _ = bf.attention(_tolist(ql), _tolist(k), _tolist(v), sc,
                             lambda i, j: j <= i and (j in sel_of_tile.get(i // tile, set()) or j >= i - W + 1))
        np.testing.assert_allclose(res["o_layers"][l], np.array([Ob[i] for i in rows_ref]), atol=1e-12)


def test_hysparse2_block_reductions():
    """k >= L selects every causal token, so each sparse layer is full causal
    attention of its own query; k = 0 selects nothing, so it is pure window
    attention over the shared K/V (both spec invariants, at block level)."""
    q0, k, v, sc = _case(L=70, Hq=4, Hkv=1, D=8, seed=64)
    q1 = _rand((70, 4, 8), 65)
    tile, W = 16, 8
    tiles = [3, 1, 4]
    full = oracle.hysparse2_block([q0, q1], k, v, sc, tile, 70, W, tiles=tiles)
    Of, _ = oracle.full_attention(q1, k, v, sc, rows=full["rows"])
    np.testing.assert_allclose(full["o_layers"][0], Of, atol=1e-13)
    none = oracle.hysparse2_block([q0, q1], k, v, sc, tile, 0, W, tiles=tiles)
    Ow, _ = oracle.window_attention(q1, k, v, sc, W, rows=none["rows"])
    np.testing.assert_allclose(none["o_layers"][0], Ow, atol=1e-13)
    assert (none["count"] == 0).all()
