"""Helpers shared by the GPU parity tests: comparison rules and input plumbing.

Comparison rules (GPU vs the fp64 oracle):
  outputs   max |gpu - oracle| <= 2e-2 for bf16 inputs, <= 1e-4 for fp32 inputs,
            and <= 1e-2 (bf16) / 1e-5 (fp32) times the oracle's largest |value|
  gradients max |gpu - oracle| <= 1e-2 times the oracle's largest |value| of
            the compared tensor, plus 1e-5 (bf16 inputs)
  scores    -inf positions identical; finite entries within 1e-4
  top-k     the index sets agree except inside the oracle's tie band: with s_k
            the oracle's k-th score and band = {c : |x_c - s_k| < 1e-4},
            oracle \\ band must be chosen by the GPU and GPU \\ oracle must lie
            in the band; set sizes and the -1 padding must match.
"""
import os

import numpy as np
import torch

import oracle

TOL_OUT = {"bf16": 2e-2, "f32": 1e-4}
# relative to the largest |reference| of the compared tensor: bf16 rounding of
# the probabilities before P V and of the output each cost up to 2^-9 of it
# (measured worst on every GPU case: 3.6e-3 bf16, 4.5e-7 fp32)
REL_OUT = {"bf16": 1e-2, "f32": 1e-5}
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
    err = float(np.max(np.abs(a - b)))
    log = os.environ.get("HYS_PARITY_LOG")
    if log:   # diagnostic: the error next to the reference's scale, per comparison
        with open(log, "a") as f:
            f.write(f"{os.environ.get('PYTEST_CURRENT_TEST', '?')}\t{err:.3e}\t{float(np.max(np.abs(b))):.3e}\n")
    return err


def check_out(gpu, ref, dtype="bf16", what=""):
    """Output parity: max |gpu - ref| within TOL_OUT[dtype] and within
    REL_OUT[dtype] of the reference's largest magnitude (an all-zero reference
    must be matched exactly, up to 1e-7)."""
    err = max_abs(gpu, ref)
    scale = float(np.max(np.abs(np.asarray(ref, dtype=np.float64)))) if np.size(ref) else 0.0
    assert err <= TOL_OUT[dtype], f"{what} error {err} above {TOL_OUT[dtype]}"
    assert err <= REL_OUT[dtype] * scale + 1e-7, f"{what} error {err} above {REL_OUT[dtype]} x {scale}"
    return err


# Gradients sum up to L terms per element (dK, dV over the query rows that see
# a key, dQ over its visible keys), so their magnitude grows with the sequence
# and a fixed absolute bound does not fit them.  The backward rounds P and dS
# to bf16 (relative error up to 2^-9 each, as the forward rounds P) before
# their products, the upstream gradient's branch split g dO to bf16, and
# accumulates in fp32; the error of each element is then a few 2^-9 of the sum
# of its terms' magnitudes, bounded here relative to the tensor's largest
# magnitude.
REL_GRAD = 1e-2
# Floor for references that vanish exactly (one visible key: dS = dP - rowsum(dO O)
# = 0): the GPU's dP and rowsum are fp32 sums of D products of order one, whose
# difference keeps a cancellation residual of order D * 2^-24.
ABS_GRAD_FLOOR = 1e-5


def check_grad(gpu, ref, what=""):
    """Gradient parity: max |gpu - ref| within REL_GRAD of the reference's largest
    magnitude, plus ABS_GRAD_FLOOR."""
    err = max_abs(gpu, ref)
    scale = float(np.max(np.abs(np.asarray(ref, dtype=np.float64)))) if np.size(ref) else 0.0
    assert err <= REL_GRAD * scale + ABS_GRAD_FLOOR, f"{what} error {err} above {REL_GRAD} x {scale} + {ABS_GRAD_FLOOR}"
    return err


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


def selection_to_compare(gpu_row, ref_row, ref_scores, k):
    """The index set a sparse-layer comparison recomputes the oracle with.

    The GPU's selection has already passed the band rule (check_topk_band).
    Where it equals the oracle's, the oracle's own end-to-end result applies;
    where it differs inside the tie band, both choices are correct and the
    oracle is re-evaluated on the GPU's choice, so the sparse layers are
    compared on every row either way.  Returns (selection, same)."""
    gpu_row = np.asarray(gpu_row)
    same = np.array_equal(gpu_row, np.asarray(ref_row))
    assert same or topk_band_ok(gpu_row, ref_row, ref_scores, k)
    return (np.asarray(ref_row) if same else gpu_row.astype(np.int64)), same
