"""Helpers shared by the GPU parity tests: comparison rules and input plumbing.

Comparison rules (GPU vs the fp64 oracle):
  outputs   max |gpu - oracle| <= 2e-2 for bf16 inputs, <= 1e-4 for fp32 inputs
  scores    -inf positions identical; finite entries within 1e-4
  top-k     the index sets agree except inside the oracle's tie band: with s_k
            the oracle's k-th score and band = {c : |x_c - s_k| < 1e-4},
            oracle \\ band must be chosen by the GPU and GPU \\ oracle must lie
            in the band; set sizes and the -1 padding must match.
"""
import numpy as np
import torch

import oracle

TOL_OUT = {"bf16": 2e-2, "f32": 1e-4}
TOL_SCORE = 1e-4
TOPK_BAND = 1e-4


def dev(t):
    return t.to("cuda")


def f64(t, dtype="bf16", scale=1.0):
    return oracle.as_f64(t, dtype, scale)


def max_abs(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    if a.size == 0:
        return 0.0
    return float(np.max(np.abs(a - b)))


def check_scores(gpu, ref, tol=TOL_SCORE):
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert gpu.shape == ref.shape, (gpu.shape, ref.shape)
    gi, ri = np.isneginf(gpu), np.isneginf(ref)
    assert np.array_equal(gi, ri), f"-inf pattern differs at {np.argwhere(gi != ri)[:5].tolist()}"
    assert not np.isnan(gpu).any()
    fin = ~ri
    err = max_abs(gpu[fin], ref[fin])
    assert err <= tol, f"score error {err}"
    return err


def topk_band_ok(gpu_row, ref_row, ref_scores, k, band=TOPK_BAND):
    """True if gpu_row is an acceptable top-k for ref_scores (see module doc)."""
    g = [int(x) for x in gpu_row if x >= 0]
    r = [int(x) for x in ref_row if x >= 0]
    if len(g) != len(r):
        return False
    if list(gpu_row[len(g):]) != [-1] * (len(gpu_row) - len(g)):
        return False
    if g != sorted(g) or len(set(g)) != len(g):
        return False
    gs, rs = set(g), set(r)
    if gs == rs:
        return True
    if len(r) < k:          # fewer valid candidates than k: sets must be equal
        return False
    sk = min(ref_scores[c] for c in r)
    inband = {c for c in range(len(ref_scores)) if abs(ref_scores[c] - sk) < band}
    return (rs - inband) <= gs and (gs - rs) <= inband


def check_topk_band(gpu_idx, ref_idx, ref_scores, k):
    """Returns (#rows identical, #rows differing inside the band); asserts none fail."""
    same = inband = 0
    bad = []
    for r in range(gpu_idx.shape[0]):
        if np.array_equal(gpu_idx[r], ref_idx[r]):
            same += 1
        elif topk_band_ok(gpu_idx[r], ref_idx[r], ref_scores[r], k):
            inband += 1
        else:
            bad.append(r)
    assert not bad, f"top-k rows outside the tie band: {bad[:10]}"
    return same, inband
