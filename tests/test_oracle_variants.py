"""Pins of the ablation-variant oracle functions (per-KV-group selection,
HySparse2 with a gated window branch, block-level selection at the token
budget).  Each reduces to an independently pinned function in a special case
or satisfies an identity with one, and tiny cases are checked by brute force.
"""
import math

import numpy as np

from oracle import hysparse as hs


def _qkv(L, Hq, Hkv, D, seed):
    r = np.random.default_rng(seed)
    return r.standard_normal((L, Hq, D)), r.standard_normal((L, Hkv, D)), r.standard_normal((L, Hkv, D))


def test_per_group_scores_max_is_the_shared_score():
    q, k, _ = _qkv(150, 8, 4, 16, 1)
    Mg = hs.block_scores_per_group(q, k, 0.25, 64)
    M = hs.block_scores(q, k, 0.25, 64)
    assert Mg.shape == (4,) + M.shape
    np.testing.assert_array_equal(Mg.max(axis=0), M)
    q1, k1, _ = _qkv(70, 4, 1, 8, 2)
    np.testing.assert_array_equal(hs.block_scores_per_group(q1, k1, 0.5, 64)[0], hs.block_scores(q1, k1, 0.5, 64))


def test_per_group_scores_brute_force():
    L, Hq, Hkv, D, blk = 9, 4, 2, 3, 4
    q, k, _ = _qkv(L, Hq, Hkv, D, 3)
    Mg = hs.block_scores_per_group(q, k, 0.7, blk)
    G = Hq // Hkv
    for g in range(Hkv):
        for i in range(L):
            for c in range((L + blk - 1) // blk):
                best = -math.inf
                for h in range(g * G, (g + 1) * G):
                    for j in range(c * blk, min(L, (c + 1) * blk)):
                        if j <= i:
                            best = max(best, 0.7 * sum(q[i, h, d] * k[j, g, d] for d in range(D)))
                assert (best == -math.inf and Mg[g, i, c] == -math.inf) or abs(Mg[g, i, c] - best) < 1e-12


def test_grouped_sparse_with_equal_sets_is_the_shared_branch():
    q, k, v = _qkv(200, 8, 2, 16, 4)
    M = hs.block_scores(q, k, 0.25, 64)
    sel, _ = hs.topk_rows(M, 2)
    o, lse = hs.sparse_block_attention(q, k, v, 0.25, sel, 64)
    og, lseg = hs.sparse_block_attention_grouped(q, k, v, 0.25, np.stack([sel, sel]), 64)
    np.testing.assert_allclose(og, o, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lseg, lse, rtol=0, atol=1e-12)


def test_grouped_sparse_brute_force():
    L, Hq, Hkv, D, blk = 10, 4, 2, 3, 4
    q, k, v = _qkv(L, Hq, Hkv, D, 5)
    sel_g = np.array([[[0, 2]] * L, [[1, -1]] * L])        # group 0: blocks 0, 2; group 1: block 1
    O, _ = hs.sparse_block_attention_grouped(q, k, v, 0.6, sel_g, blk)
    G = Hq // Hkv
    for i in range(L):
        for h in range(Hq):
            g = h // G
            J = [j for j in range(i + 1) if j // blk in [c for c in sel_g[g][i] if c >= 0]]
            if not J:
                assert np.all(O[i, h] == 0)
                continue
            s = [0.6 * sum(q[i, h, d] * k[j, g, d] for d in range(D)) for j in J]
            m = max(s)
            w = [math.exp(x - m) for x in s]
            for d in range(D):
                ref = sum(wi * v[j, g, d] for wi, j in zip(w, J)) / sum(w)
                assert abs(O[i, h, d] - ref) < 1e-12


def test_gated_window_special_cases():
    L, Hq, Hkv, D, tile, W = 200, 4, 1, 16, 64, 128
    q, k, v = _qkv(L, Hq, Hkv, D, 6)
    T = hs.tile_token_scores(q, k, 0.25, tile)
    sel, _ = hs.topk_rows(T, 32)
    # zero gate weights: g = 1/2, the plain average of the two branches
    # (rows whose selected set is empty take the window branch alone)
    o = hs.hysparse2_gated_window_layer(q, k, v, 0.25, sel, tile, W, np.zeros((Hq, D)))
    o_sp, lse_sp = hs.sparse_token_attention(q, k, v, 0.25, sel, tile, 0)
    o_w, _ = hs.window_attention(q, k, v, 0.25, W)
    live = np.isfinite(lse_sp.T)                               # [L, Hq]
    assert live.any() and (~live).any()
    np.testing.assert_allclose(o[live], 0.5 * (o_sp + o_w)[live], rtol=0, atol=1e-12)
    np.testing.assert_allclose(o[~live], o_w[~live], rtol=0, atol=1e-12)
    # a saturated gate picks one branch: with q[..., 0] = 1 and w = +-60 e_0,
    # g = sigmoid(+-60) is 1 (sparse branch) or 0 (window branch) to 1e-26
    q1 = q.copy()
    q1[:, :, 0] = 1.0
    T1 = hs.tile_token_scores(q1, k, 0.25, tile)
    sel1, _ = hs.topk_rows(T1, 32)
    o_sp1, lse_sp1 = hs.sparse_token_attention(q1, k, v, 0.25, sel1, tile, 0)
    o_w1, _ = hs.window_attention(q1, k, v, 0.25, W)
    live1 = np.isfinite(lse_sp1.T)
    e0 = np.zeros((Hq, D))
    e0[:, 0] = 60.0
    o = hs.hysparse2_gated_window_layer(q1, k, v, 0.25, sel1, tile, W, e0)
    np.testing.assert_allclose(o[live1], o_sp1[live1], rtol=0, atol=1e-12)
    np.testing.assert_allclose(o[~live1], o_w1[~live1], rtol=0, atol=1e-12)
    o = hs.hysparse2_gated_window_layer(q1, k, v, 0.25, sel1, tile, W, -e0)
    np.testing.assert_allclose(o, o_w1, rtol=0, atol=1e-12)
    # nothing selected: the window branch alone
    none = np.full_like(sel, -1)
    o = hs.hysparse2_gated_window_layer(q, k, v, 0.25, none, tile, W, np.ones((Hq, D)))
    np.testing.assert_allclose(o, o_w, rtol=0, atol=1e-12)


def test_tile_block_scores_are_the_tile_max_of_block_scores():
    # a tile's block score is the max over its query rows of the per-query block scores
    L, tile = 260, 64
    q, k, _ = _qkv(L, 4, 2, 16, 7)
    T = hs.tile_token_scores(q, k, 0.25, tile)
    Mt = hs.tile_block_scores(T, 64)
    M = hs.block_scores(q, k, 0.25, 64)
    for t in range(T.shape[0]):
        np.testing.assert_allclose(Mt[t], M[t * tile:min(L, (t + 1) * tile)].max(axis=0), rtol=0, atol=1e-12)


def test_expand_blocks():
    e = hs.expand_blocks(np.array([[0, 2, -1], [3, -1, -1]]), 4, 14)
    assert e[0].tolist() == [0, 1, 2, 3, 8, 9, 10, 11, -1, -1, -1, -1]
    assert e[1].tolist() == [12, 13] + [-1] * 10                # the last block is cut at Lk
