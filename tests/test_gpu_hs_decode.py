"""GPU parity of hys_hysparse_decode_step (HySparse decode with ring window caches) against the oracle.

Rules (tests/parity_util.py): outputs within 2e-2 max-abs and within 1e-2 of
the oracle's largest magnitude (bf16 inputs; decode outputs are small, so the
relative rule is the binding one);
block scores with the oracle's -inf pattern and 1e-4 elsewhere; the selected
blocks equal to the oracle's (random inputs, no ties at the k-th score); the
rings bit-exact: the new token's K/V in slot (n-1) mod W, every other slot
unchanged.  Lengths cover n = 1, n below W, wrap-around and block edges; a
second step on the updated rings checks that the ring carries over.
"""
import math

import numpy as np
import pytest
import torch

import synth
from hybrid_sparse_attention_flash_amd import ops
from oracle.hysparse_decode import hysparse_decode_step
from tests.parity_util import check_out, check_scores

pytestmark = pytest.mark.gpu


def f64(t):
    return t.to(torch.float64).numpy()


def _oracle(x, w, lens, topk, scale, rings_k=None, rings_v=None):
    rk = rings_k if rings_k is not None else [f64(r) for r in x["k_ring"]]
    rv = rings_v if rings_v is not None else [f64(r) for r in x["v_ring"]]
    out = []
    for b in range(w.B):
        out.append(hysparse_decode_step(
            f64(x["q_full"][b, 0]), f64(x["k"][b]), f64(x["v"][b]), scale, lens[b], w.L,
            [f64(q[b, 0]) for q in x["q"]], [r[b] for r in rk], [r[b] for r in rv],
            [f64(t[b, 0]) for t in x["k_new"]], [f64(t[b, 0]) for t in x["v_new"]],
            [g.numpy().astype(np.float64) for g in x["gate_w"]], 64, topk))
    return out


def _gpu(x, w, lens, topk, out_dtype, rings=None):
    B, Hq, D = w.B, w.Hq, w.D
    nblk = (w.L + 63) // 64
    dev = "cuda"
    kr = rings[0] if rings else [r.to(dev) for r in x["k_ring"]]
    vr = rings[1] if rings else [r.to(dev) for r in x["v_ring"]]
    o_full = torch.empty(B, 1, Hq, D, dtype=out_dtype, device=dev)
    bs = torch.empty(B, nblk, dtype=torch.float32, device=dev)
    idx = torch.empty(B, topk, dtype=torch.int32, device=dev)
    o_sp = [torch.empty(B, 1, Hq, D, dtype=out_dtype, device=dev) for _ in x["q"]]
    ops.hys_hysparse_decode_step(
        x["q_full"].to(dev), x["k"].to(dev), x["v"].to(dev), lens, o_full, bs, idx,
        [q.to(dev) for q in x["q"]], [t.to(dev) for t in x["k_new"]], [t.to(dev) for t in x["v_new"]],
        kr, vr, [g.to(dev) for g in x["gate_w"]], o_sp, topk)
    torch.cuda.synchronize()
    return o_full, bs, idx, o_sp, kr, vr


def _check(x, w, lens, topk, ref, got, before_k, before_v):
    o_full, bs, idx, o_sp, kr, vr = got
    W = w.window
    for b in range(w.B):
        r = ref[b]
        check_out(o_full[b, 0].float().cpu().numpy(), r["o_full"], "bf16", f"o_full {b}")
        check_scores(bs[b].cpu().numpy(), r["block_scores"])
        assert idx[b].cpu().tolist() == r["sel"].tolist(), (b, idx[b].cpu().tolist(), r["sel"].tolist())
        for l in range(len(o_sp)):
            check_out(o_sp[l][b, 0].float().cpu().numpy(), r["o_layers"][l], "bf16", f"o_sparse {b} {l}")
        slot = (lens[b] - 1) % W
        for l in range(len(kr)):
            for ring, before, new in ((kr[l], before_k[l], x["k_new"][l]), (vr[l], before_v[l], x["v_new"][l])):
                got_r = ring[b].cpu()
                assert torch.equal(got_r[slot], new[b, 0]), (b, l)
                keep = [s for s in range(W) if s != slot]
                assert torch.equal(got_r[keep], before[b][keep]), (b, l)


CASES = [
    # B, N, lens, Hq, Hkv, D, topk, n_sparse, out dtype
    (2, 700, (700, 129), 8, 2, 128, 3, 2, torch.bfloat16),
    (3, 300, (1, 64, 300), 16, 1, 64, 5, 1, torch.float32),
    (1, 5000, (4097,), 32, 4, 128, 16, 3, torch.float32),
    (2, 1000, (128, 577), 32, 8, 128, 4, 2, torch.bfloat16),
]


@pytest.mark.parametrize("B,N,lens,Hq,Hkv,D,topk,nsp,odt", CASES)
def test_hysparse_decode_step(B, N, lens, Hq, Hkv, D, topk, nsp, odt):
    w = synth.HS_DECODE_WORKLOAD.shrink(B=B, L=N, Hq=Hq, Hkv=Hkv, D=D, n_sparse=nsp, topk=topk)
    x = synth.gen_hs_decode(w, seed=N)
    scale = 1.0 / math.sqrt(D)
    ref = _oracle(x, w, list(lens), topk, scale)
    got = _gpu(x, w, list(lens), topk, odt)
    _check(x, w, list(lens), topk, ref, got, x["k_ring"], x["v_ring"])


def test_hysparse_decode_two_steps_carry_the_ring():
    """Step n, then step n+1 on the rings the first step updated."""
    w = synth.HS_DECODE_WORKLOAD.shrink(B=2, L=400, Hq=8, Hkv=2, D=128, n_sparse=2, topk=4)
    x = synth.gen_hs_decode(w, seed=5)
    scale = 1.0 / math.sqrt(w.D)
    lens = [300, 128]
    ref1 = _oracle(x, w, lens, w.topk, scale)
    got1 = _gpu(x, w, lens, w.topk, torch.float32)
    _check(x, w, lens, w.topk, ref1, got1, x["k_ring"], x["v_ring"])
    # second step: new queries and new window K/V, one more token in the cache
    x2 = synth.gen_hs_decode(w, seed=6)
    x2["k"], x2["v"], x2["k_ring"], x2["v_ring"] = x["k"], x["v"], [r.cpu() for r in got1[4]], [r.cpu() for r in got1[5]]
    lens2 = [n + 1 for n in lens]
    rk = [np.stack([ref1[b]["rings"][l][0] for b in range(w.B)]) for l in range(w.n_sparse)]
    rv = [np.stack([ref1[b]["rings"][l][1] for b in range(w.B)]) for l in range(w.n_sparse)]
    ref2 = _oracle(x2, w, lens2, w.topk, scale, rk, rv)
    before_k = [r.clone() for r in x2["k_ring"]]
    before_v = [r.clone() for r in x2["v_ring"]]
    got2 = _gpu(x2, w, lens2, w.topk, torch.float32, rings=(got1[4], got1[5]))
    _check(x2, w, lens2, w.topk, ref2, got2, before_k, before_v)


def test_hysparse_decode_full_size():
    """The 128k workload at its full size (B=4, 32/4 heads, 11 sparse layers), every output checked."""
    w = synth.HS_DECODE_WORKLOAD
    x = synth.gen_hs_decode(w, seed=0)
    lens = w.lens()
    ref = _oracle(x, w, lens, w.topk, 1.0 / math.sqrt(w.D))
    got = _gpu(x, w, lens, w.topk, torch.bfloat16)
    _check(x, w, lens, w.topk, ref, got, x["k_ring"], x["v_ring"])
