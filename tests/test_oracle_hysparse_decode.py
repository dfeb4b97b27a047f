"""Pins of the HySparse decode-step oracle (ring window caches, block scores).

The decode step must reproduce the prefill hybrid block (pinned on its own in
test_oracle.py) at the last row n-1: the same full-layer output, the same
block scores, the same selection and the same gated sparse-layer outputs,
with the window taken from a ring instead of the window K/V tensor.  The
cache beyond n and every ring slot outside the window hold NaN, so any read
of them would show.  Lengths cover n < W, n = W, wrap-around and block edges.
"""
import numpy as np
import pytest

from oracle import hysparse as hs
from oracle.hysparse_decode import (block_scores_decode, hysparse_decode_step, ring_append, ring_slot,
                                    ring_window)


def _case(n, nmax, Hq=8, Hkv=2, D=16, nl=2, W=128, seed=0):
    rng = np.random.default_rng(seed)
    q_layers = [rng.standard_normal((n, Hq, D)) for _ in range(nl + 1)]
    k = rng.standard_normal((n, Hkv, D))
    v = rng.standard_normal((n, Hkv, D))
    kw = [rng.standard_normal((n, Hkv, D)) for _ in range(nl)]
    vw = [rng.standard_normal((n, Hkv, D)) for _ in range(nl)]
    gw = [0.3 * rng.standard_normal((Hq, D)) for _ in range(nl)]
    kc = np.full((nmax, Hkv, D), np.nan)
    vc = np.full((nmax, Hkv, D), np.nan)
    kc[:n], vc[:n] = k, v
    rings_k, rings_v = [], []
    for l in range(nl):
        rk = np.full((W, Hkv, D), np.nan)
        rv = np.full((W, Hkv, D), np.nan)
        for t in range(max(0, n - W), n - 1):      # the ring before the step: tokens up to n-2
            rk[t % W], rv[t % W] = kw[l][t], vw[l][t]
        rings_k.append(rk)
        rings_v.append(rv)
    return q_layers, k, v, kw, vw, gw, kc, vc, rings_k, rings_v


@pytest.mark.parametrize("n", [1, 5, 63, 64, 65, 128, 129, 300, 511])
def test_decode_step_equals_prefill_last_row(n):
    nmax, block, topk, W, scale = 520, 64, 3, 128, 0.25
    q_layers, k, v, kw, vw, gw, kc, vc, rk, rv = _case(n, nmax, seed=n)
    ref = hs.hysparse_block(q_layers, k, v, kw, vw, gw, scale, block, topk, W, rows=[n - 1])
    dec = hysparse_decode_step(q_layers[0][n - 1], kc, vc, scale, n, nmax,
                               [q[n - 1] for q in q_layers[1:]], rk, rv,
                               [x[n - 1] for x in kw], [x[n - 1] for x in vw], gw, block, topk)
    np.testing.assert_allclose(dec["o_full"], ref["o_full"][0], rtol=0, atol=1e-12)
    nb = (n + block - 1) // block
    np.testing.assert_allclose(dec["block_scores"][:nb], ref["scores"][0], rtol=0, atol=1e-12)
    assert np.all(dec["block_scores"][nb:] == -np.inf)
    assert dec["sel"].tolist() == ref["sel"][0].tolist() and dec["count"] == ref["count"][0]
    for l in range(len(gw)):
        np.testing.assert_allclose(dec["o_layers"][l], ref["o_layers"][l][0], rtol=0, atol=1e-12)
        assert not np.isnan(dec["o_layers"][l]).any()


def test_ring_slots_append_and_window_order():
    W, Hkv, D = 4, 1, 1
    ring = np.full((W, Hkv, D), -1.0)
    for t in range(9):                               # tokens 0..8 written as they arrive
        ring[ring_slot(t, W)] = t
    rk, rv = ring_append(ring, ring, np.array([[9.0]]), np.array([[9.0]]), n=10)
    assert ring_slot(9, W) == 1 and rk[1, 0, 0] == 9.0 and ring[1, 0, 0] == 5.0   # a copy is returned
    kw, vw, pos = ring_window(rk, rv, n=10)
    assert pos.tolist() == [6, 7, 8, 9] and kw[:, 0, 0].tolist() == [6.0, 7.0, 8.0, 9.0]
    # short sequence: the window is every token so far
    kw, _, pos = ring_window(rk, rv, n=3)
    assert pos.tolist() == [0, 1, 2]


def test_block_scores_decode_blocks_and_tail():
    s = np.arange(150, dtype=np.float64)
    s[70] = 1000.0
    M = block_scores_decode(s, n=130, block=64, nblk=4)
    assert M.tolist() == [63.0, 1000.0, 129.0, -np.inf]   # keys >= n are ignored


def test_window_with_empty_selection_is_the_window_branch():
    # topk = 0 selects nothing: every sparse layer returns its window branch
    n, nmax, W = 200, 256, 128
    q_layers, k, v, kw, vw, gw, kc, vc, rk, rv = _case(n, nmax, seed=3)
    dec = hysparse_decode_step(q_layers[0][n - 1], kc, vc, 0.25, n, nmax, [q[n - 1] for q in q_layers[1:]],
                               rk, rv, [x[n - 1] for x in kw], [x[n - 1] for x in vw], gw, 64, 0)
    for l in range(len(gw)):
        o_w, _ = hs.window_attention(q_layers[l + 1], kw[l], vw[l], 0.25, W, rows=[n - 1])
        np.testing.assert_allclose(dec["o_layers"][l], o_w[0], rtol=0, atol=1e-12)
