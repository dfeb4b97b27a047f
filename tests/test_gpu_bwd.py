"""GPU parity of the backward pass against the oracle (oracle/hysparse_bwd.py).

Inputs are bf16 (q, k, v, window K/V, upstream gradients) with fp32 gate
weights; the oracle differentiates the fp64 forward on the same values.
Gradients follow the gradient rule of tests/parity_util.py (1e-2 of the
reference's largest magnitude: the GPU rounds P and dS to bf16 before their
products, as the forward rounds P; gradients are sums over up to L terms, so
no fixed absolute bound fits them); the window forward follows the output
rule.  Selections are seeded random block sets (distinct causal blocks per row, some rows empty) given to
both sides; the block-level test runs the whole training step on the GPU and
checks its selection bit-exact against the oracle's before comparing
gradients.  Sizes span several 128-key and 64-query tiles with ragged tails,
G = 1, 2, 4 and 8, both head dims, and a length whose dK/dV pass splits the
query rows of a key tile over several workgroups (more than 64 row blocks).
"""
import math

import numpy as np
import pytest
import torch

import oracle
import synth
from oracle import hysparse_bwd as hb
from hybrid_sparse_attention_flash_amd import ops
from hybrid_sparse_attention_flash_amd.block import HySparseTrainer
from tests.parity_util import check_grad, check_out

pytestmark = pytest.mark.gpu


def _bf(rng, *shape, s=1.0):
    return torch.from_numpy((s * rng.standard_normal(shape)).astype(np.float32)).to(torch.bfloat16)


def _f64(t):
    return t.to(torch.float64).numpy()


def _rand_sel(rng, L, k, empty_every=0):
    """Per row: up to k distinct blocks among the causal ones, ascending, -1 padded."""
    sel = np.full((L, k), -1, dtype=np.int32)
    for i in range(L):
        if empty_every and i % empty_every == 3:
            continue
        nb = i // 64 + 1
        ch = np.sort(rng.choice(nb, size=min(k, nb), replace=False))
        sel[i, :len(ch)] = ch
    return sel


FULL_CASES = [
    # B, L, Hq, Hkv, D
    (1, 300, 8, 2, 128),
    (2, 200, 4, 4, 64),
    (1, 520, 8, 1, 64),
    (1, 129, 2, 1, 128),
    (1, 2300, 4, 1, 64),       # more than 64 row blocks: the dK/dV rows split over two workgroups
    (2, 1, 4, 2, 128),         # one token
    (1, 64, 8, 1, 64),         # exactly one key block
    (1, 333, 12, 1, 128),      # G = 12: dQ workgroups of 16 rows x 8 heads, the second head chunk half empty
    (2, 150, 16, 1, 64),       # G = 16: two full head chunks
    (2, 77, 8, 2, 128),        # G = 8, two sequences, 16-row blocks with a ragged tail
]


@pytest.mark.parametrize("B,L,Hq,Hkv,D", FULL_CASES)
def test_full_attn_bwd(B, L, Hq, Hkv, D):
    rng = np.random.default_rng(L + Hq)
    q, k, v = _bf(rng, B, L, Hq, D), _bf(rng, B, L, Hkv, D), _bf(rng, B, L, Hkv, D)
    do = _bf(rng, B, L, Hq, D)
    scale = 1.0 / math.sqrt(D)
    dev = "cuda"
    qd, kd, vd, dod = q.to(dev), k.to(dev), v.to(dev), do.to(dev)
    o = torch.empty(B, L, Hq, D, dtype=torch.float32, device=dev)
    lse = torch.empty(B, Hq, L, dtype=torch.float32, device=dev)
    ops.hys_full_attn_fwd(qd, kd, vd, o, lse)
    dq = torch.empty(B, L, Hq, D, dtype=torch.float32, device=dev)
    dk = torch.full((B, L, Hkv, D), 7.0, dtype=torch.float32, device=dev)     # overwritten
    dv = torch.full((B, L, Hkv, D), 7.0, dtype=torch.float32, device=dev)
    ops.hys_full_attn_bwd(qd, kd, vd, o, lse, dod, dq, dk, dv)
    torch.cuda.synchronize()
    for b in range(B):
        rq, rk, rv = hb.full_attention_bwd(_f64(q[b]), _f64(k[b]), _f64(v[b]), scale, _f64(do[b]))
        check_grad(dq[b].cpu().numpy(), rq, "dq")
        check_grad(dk[b].cpu().numpy(), rk, "dk")
        check_grad(dv[b].cpu().numpy(), rv, "dv")
    # accumulate: a second call adds the same gradient
    ops.hys_full_attn_bwd(qd, kd, vd, o, lse, dod, dq, dk, dv, accumulate_kv=True)
    torch.cuda.synchronize()
    rq, rk, rv = hb.full_attention_bwd(_f64(q[0]), _f64(k[0]), _f64(v[0]), scale, _f64(do[0]))
    check_grad(dk[0].cpu().numpy(), 2 * rk, "dk accumulated")
    check_grad(dv[0].cpu().numpy(), 2 * rv, "dv accumulated")


@pytest.mark.parametrize("L,Hq,Hkv,D,W", [(300, 8, 2, 128, 128), (200, 4, 1, 64, 37)])
def test_window_attn_fwd(L, Hq, Hkv, D, W):
    rng = np.random.default_rng(5)
    q, kw, vw = _bf(rng, 1, L, Hq, D), _bf(rng, 1, L, Hkv, D), _bf(rng, 1, L, Hkv, D)
    o = torch.empty(1, L, Hq, D, dtype=torch.float32, device="cuda")
    lse = torch.empty(1, Hq, L, dtype=torch.float32, device="cuda")
    ops.hys_window_attn_fwd(q.cuda(), kw.cuda(), vw.cuda(), W, o, lse)
    torch.cuda.synchronize()
    O, LSE = oracle.window_attention(_f64(q[0]), _f64(kw[0]), _f64(vw[0]), 1.0 / math.sqrt(D), W)
    check_out(o[0].cpu().numpy(), O, "bf16", "window o")
    assert np.abs(lse[0].cpu().numpy() - LSE).max() <= 1e-3


SPARSE_CASES = [
    # B, L, Hq, Hkv, D, k, window, per-group sets, dO fp32
    (1, 330, 8, 2, 128, 3, 128, False, False),
    (2, 200, 4, 1, 64, 2, 50, False, True),
    (1, 300, 16, 4, 128, 2, 128, True, False),
    (1, 260, 8, 8, 64, 4, 64, True, True),
    (1, 2300, 4, 2, 64, 3, 128, False, False),     # split dK/dV rows
    (1, 270, 16, 2, 128, 3, 128, True, False),     # G = 8: 16-row dQ workgroups, per-group unions
    (1, 150, 12, 1, 64, 2, 64, False, True),       # G = 12: a partly empty head chunk
    (2, 100, 8, 1, 64, 2, 32, False, True),        # G = 8, two sequences, L not a multiple of 16
]


@pytest.mark.parametrize("B,L,Hq,Hkv,D,kb,W,grouped,do32", SPARSE_CASES)
def test_sparse_layer_bwd(B, L, Hq, Hkv, D, kb, W, grouped, do32):
    rng = np.random.default_rng(L * 7 + Hq)
    scale = 1.0 / math.sqrt(D)
    q, k, v = _bf(rng, B, L, Hq, D), _bf(rng, B, L, Hkv, D), _bf(rng, B, L, Hkv, D)
    kw, vw = _bf(rng, B, L, Hkv, D), _bf(rng, B, L, Hkv, D)
    gw = torch.from_numpy((0.3 * rng.standard_normal((Hq, D))).astype(np.float32))
    do = torch.from_numpy(rng.standard_normal((B, L, Hq, D)).astype(np.float32))
    do = do if do32 else do.to(torch.bfloat16)
    ng = Hkv if grouped else 1
    sel = np.stack([np.stack([_rand_sel(rng, L, kb, empty_every=11) for _ in range(B)]) for _ in range(ng)])
    dev = "cuda"
    idx = torch.from_numpy(sel).to(dev)                     # [ng, B, L, kb]
    idx_arg = idx if grouped else idx[0]
    qd, kd, vd, kwd, vwd, gwd, dod = (t.to(dev) for t in (q, k, v, kw, vw, gw, do))
    f32 = dict(dtype=torch.float32, device=dev)
    o_sp, lse_sp = torch.empty(B, L, Hq, D, **f32), torch.empty(B, Hq, L, **f32)
    o_w, lse_w = torch.empty(B, L, Hq, D, **f32), torch.empty(B, Hq, L, **f32)
    ops.hys_sparse_attn_fwd(qd, kd, vd, idx_arg, o_sp, lse_sp, granularity=64, topk=kb)
    ops.hys_window_attn_fwd(qd, kwd, vwd, W, o_w, lse_w)
    dq = torch.empty(B, L, Hq, D, **f32)
    dk, dv = torch.ones(B, L, Hkv, D, **f32), torch.ones(B, L, Hkv, D, **f32)     # accumulated into
    dkw, dvw = torch.empty(B, L, Hkv, D, **f32), torch.empty(B, L, Hkv, D, **f32)
    dgw = torch.empty(Hq, D, **f32)
    ops.hys_sparse_layer_bwd(qd, kd, vd, idx_arg, kwd, vwd, W, gwd, o_sp, lse_sp, o_w, lse_w, dod, dq, dk, dv, dkw,
                             dvw, dgw, accumulate_kv=True, topk=kb)
    torch.cuda.synchronize()
    dgw_ref = np.zeros((Hq, D))
    for b in range(B):
        r = hb.sparse_layer_bwd(_f64(q[b]), _f64(k[b]), _f64(v[b]), _f64(kw[b]), _f64(vw[b]),
                                gw.numpy().astype(np.float64), scale, sel[0, b], 64, W, do[b].double().numpy(),
                                sel_groups=sel[:, b] if grouped else None)
        check_grad(dq[b].cpu().numpy(), r["dq"], "dq")
        check_grad(dk[b].cpu().numpy() - 1.0, r["dk"], "dk")
        check_grad(dv[b].cpu().numpy() - 1.0, r["dv"], "dv")
        check_grad(dkw[b].cpu().numpy(), r["dkw"], "dk_win")
        check_grad(dvw[b].cpu().numpy(), r["dvw"], "dv_win")
        dgw_ref += r["dgate_w"]
    check_grad(dgw.cpu().numpy(), dgw_ref, "dgate_w")


def test_hysparse_block_training_step():
    """Forward (saving the branches) and backward of a whole block on the GPU against the oracle."""
    B, L, Hq, Hkv, D, nsp, kb, W = 1, 384, 8, 2, 128, 2, 2, 128
    rng = np.random.default_rng(11)
    scale = 1.0 / math.sqrt(D)
    ql = [_bf(rng, B, L, Hq, D) for _ in range(nsp + 1)]
    k, v = _bf(rng, B, L, Hkv, D), _bf(rng, B, L, Hkv, D)
    kw = [_bf(rng, B, L, Hkv, D) for _ in range(nsp)]
    vw = [_bf(rng, B, L, Hkv, D) for _ in range(nsp)]
    gw = [torch.from_numpy((0.3 * rng.standard_normal((Hq, D))).astype(np.float32)) for _ in range(nsp)]
    do_full = _bf(rng, B, L, Hq, D)
    do_l = [_bf(rng, B, L, Hq, D) for _ in range(nsp)]
    dev = "cuda"
    cu = lambda xs: [x.to(dev) for x in xs]
    tr = HySparseTrainer(B, L, Hq, Hkv, D, nsp, kb, W, device=dev)
    args = (cu(ql), k.to(dev), v.to(dev), cu(kw), cu(vw), cu(gw))
    tr.forward(*args)
    tr.backward(*args, do_full.to(dev), cu(do_l))
    torch.cuda.synchronize()
    r = hb.hysparse_block_bwd([_f64(x[0]) for x in ql], _f64(k[0]), _f64(v[0]), [_f64(x[0]) for x in kw],
                              [_f64(x[0]) for x in vw], [g.numpy().astype(np.float64) for g in gw], scale, 64, kb, W,
                              _f64(do_full[0]), [_f64(x[0]) for x in do_l])
    assert np.array_equal(tr.fwd.idx[0, 0].cpu().numpy(), r["sel"])
    for l in range(nsp + 1):
        check_grad(tr.dq[l][0].cpu().numpy(), r["dq"][l], f"dq {l}")
    check_grad(tr.dk[0].cpu().numpy(), r["dk"], "dk (full + sparse layers)")
    check_grad(tr.dv[0].cpu().numpy(), r["dv"], "dv (full + sparse layers)")
    for l in range(nsp):
        check_grad(tr.dkw[l][0].cpu().numpy(), r["dkw"][l], f"dk_win {l}")
        check_grad(tr.dvw[l][0].cpu().numpy(), r["dvw"][l], f"dv_win {l}")
        check_grad(tr.dgate_w[l].cpu().numpy(), r["dgate_w"][l], f"dgate_w {l}")


class RowView:
    """Float64 view of a stored [L, H, D] tensor that converts only indexed rows."""

    def __init__(self, t):
        self.t = t
        self.shape = tuple(t.shape)

    def __getitem__(self, rows):
        return self.t[torch.as_tensor(np.asarray(rows))].to(torch.float64).numpy()


def test_moe80b_32k_backward_sampled():
    """The 32k HySparse block (1 full + 11 sparse layers) at its full size, in
    the launch configuration the bench times (16 row splits in the dK/dV
    pass): dq of every layer on sampled rows, and on the last 64 keys, which
    only the last 64 rows see, the shared dK/dV (full layer plus every sparse
    layer's share) and each layer's window dK/dV."""
    w = synth.WORKLOADS["moe80b_32k"]
    print("backward 32k: generating inputs", flush=True)
    q = [synth.gen_q(w, l) for l in range(w.n_sparse + 1)]
    k, v = synth.gen_kv(w, "k")[0], synth.gen_kv(w, "v")[0]
    kw = [synth.gen_window_kv(w, l + 1, "kw")[0] for l in range(w.n_sparse)]
    vw = [synth.gen_window_kv(w, l + 1, "vw")[0] for l in range(w.n_sparse)]
    gw = [synth.gen_gate_w(w, l + 1) for l in range(w.n_sparse)]
    dout = [synth.gen_grad_out(w, l) for l in range(w.n_sparse + 1)]
    dev = "cuda"
    cu = lambda xs: [x.to(dev) for x in xs]
    tr = HySparseTrainer(w.B, w.L, w.Hq, w.Hkv, w.D, w.n_sparse, w.topk, w.window, device=dev)
    args = (cu(q), k.to(dev), v.to(dev), cu(kw), cu(vw), cu(gw))
    print("backward 32k: forward and backward on the GPU", flush=True)
    tr.forward(*args)
    tr.backward(*args, dout[0].to(dev), cu(dout[1:]))
    torch.cuda.synchronize()
    L, W = w.L, w.window
    last = np.arange(L - 64, L)
    rows = np.concatenate([np.array([0, 63, 64, 5000, 20000]), last])
    kf, vf = k[0].to(torch.float64).numpy(), v[0].to(torch.float64).numpy()
    print("backward 32k: oracle selection and full layer", flush=True)
    sel, _ = oracle.topk_rows(oracle.block_scores(RowView(q[0][0]), kf, w.scale, 64, rows), w.topk)
    assert np.array_equal(tr.fwd.idx[0, 0][torch.as_tensor(rows)].cpu().numpy(), sel)
    r = torch.as_tensor(rows)
    dq0, dk, dv = hb.full_attention_bwd(RowView(q[0][0]), kf, vf, w.scale, RowView(dout[0][0]), rows=rows)
    check_grad(tr.dq[0][0][r].cpu().numpy(), dq0, "dq full layer")
    for l in range(w.n_sparse):
        print(f"backward 32k: oracle sparse layer {l}", flush=True)
        res = hb.sparse_layer_bwd(RowView(q[l + 1][0]), kf, vf, kw[l][0].to(torch.float64).numpy(),
                                  vw[l][0].to(torch.float64).numpy(), gw[l].numpy().astype(np.float64), w.scale,
                                  sel, 64, W, RowView(dout[l + 1][0]), rows=rows)
        check_grad(tr.dq[l + 1][0][r].cpu().numpy(), res["dq"], f"dq layer {l}")
        check_grad(tr.dkw[l][0][L - 64:].cpu().numpy(), res["dkw"][L - 64:], f"dk_win layer {l}")
        check_grad(tr.dvw[l][0][L - 64:].cpu().numpy(), res["dvw"][L - 64:], f"dv_win layer {l}")
        dk = dk + res["dk"]
        dv = dv + res["dv"]
    check_grad(tr.dk[0][L - 64:].cpu().numpy(), dk[L - 64:], "dk (full + 11 sparse layers)")
    check_grad(tr.dv[0][L - 64:].cpu().numpy(), dv[L - 64:], "dv (full + 11 sparse layers)")


def test_sparse_layer_bwd_gate_bias():
    """The gate with a per-head bias: dq, dgate_w and the bias gradient dgate_b."""
    B, L, Hq, Hkv, D, kb, W = 1, 330, 8, 2, 128, 3, 128
    rng = np.random.default_rng(1234)
    scale = 1.0 / math.sqrt(D)
    q, k, v = _bf(rng, B, L, Hq, D), _bf(rng, B, L, Hkv, D), _bf(rng, B, L, Hkv, D)
    kw, vw = _bf(rng, B, L, Hkv, D), _bf(rng, B, L, Hkv, D)
    gw = torch.from_numpy((0.3 * rng.standard_normal((Hq, D))).astype(np.float32))
    gb = torch.from_numpy((0.8 * rng.standard_normal(Hq)).astype(np.float32))
    do = _bf(rng, B, L, Hq, D)
    sel = _rand_sel(rng, L, kb, empty_every=11)
    dev = "cuda"
    idx = torch.from_numpy(sel)[None].to(dev)
    qd, kd, vd, kwd, vwd = (t.to(dev) for t in (q, k, v, kw, vw))
    f32 = dict(dtype=torch.float32, device=dev)
    o_sp, lse_sp = torch.empty(B, L, Hq, D, **f32), torch.empty(B, Hq, L, **f32)
    o_w, lse_w = torch.empty(B, L, Hq, D, **f32), torch.empty(B, Hq, L, **f32)
    ops.hys_sparse_attn_fwd(qd, kd, vd, idx, o_sp, lse_sp, granularity=64, topk=kb)
    ops.hys_window_attn_fwd(qd, kwd, vwd, W, o_w, lse_w)
    dq = torch.empty(B, L, Hq, D, **f32)
    dk, dv = torch.empty(B, L, Hkv, D, **f32), torch.empty(B, L, Hkv, D, **f32)
    dkw, dvw = torch.empty(B, L, Hkv, D, **f32), torch.empty(B, L, Hkv, D, **f32)
    dgw, dgb = torch.empty(Hq, D, **f32), torch.full((Hq,), 7.0, **f32)
    ops.hys_sparse_layer_bwd(qd, kd, vd, idx, kwd, vwd, W, gw.to(dev), o_sp, lse_sp, o_w, lse_w, do.to(dev), dq, dk,
                             dv, dkw, dvw, dgw, gate_b=gb.to(dev), topk=kb, dgate_b=dgb)
    torch.cuda.synchronize()
    r = hb.sparse_layer_bwd(_f64(q[0]), _f64(k[0]), _f64(v[0]), _f64(kw[0]), _f64(vw[0]), gw.numpy().astype(np.float64),
                            scale, sel, 64, W, _f64(do[0]), gate_b=gb.numpy().astype(np.float64))
    check_grad(dq[0].cpu().numpy(), r["dq"], "dq (biased gate)")
    check_grad(dk[0].cpu().numpy(), r["dk"], "dk (biased gate)")
    check_grad(dgw.cpu().numpy(), r["dgate_w"], "dgate_w (biased gate)")
    check_grad(dgb.cpu().numpy(), r["dgate_b"], "dgate_b")


@pytest.mark.parametrize("L", [64, 200])
def test_sparse_layer_bwd_empty_selection(L):
    """k = 0: no sparse branch anywhere, so every gradient is the window branch's
    and the shared K/V receive nothing (accumulated into, so they stay as given)."""
    B, Hq, Hkv, D, W = 1, 4, 2, 64, 50
    rng = np.random.default_rng(L)
    scale = 1.0 / math.sqrt(D)
    q, k, v = _bf(rng, B, L, Hq, D), _bf(rng, B, L, Hkv, D), _bf(rng, B, L, Hkv, D)
    kw, vw = _bf(rng, B, L, Hkv, D), _bf(rng, B, L, Hkv, D)
    gw = torch.from_numpy((0.3 * rng.standard_normal((Hq, D))).astype(np.float32))
    do = _bf(rng, B, L, Hq, D)
    dev = "cuda"
    idx = torch.empty(B, L, 0, dtype=torch.int32, device=dev)
    qd, kd, vd, kwd, vwd = (t.to(dev) for t in (q, k, v, kw, vw))
    f32 = dict(dtype=torch.float32, device=dev)
    o_sp, lse_sp = torch.empty(B, L, Hq, D, **f32), torch.empty(B, Hq, L, **f32)
    o_w, lse_w = torch.empty(B, L, Hq, D, **f32), torch.empty(B, Hq, L, **f32)
    ops.hys_sparse_attn_fwd(qd, kd, vd, idx, o_sp, lse_sp, granularity=64, topk=0)
    ops.hys_window_attn_fwd(qd, kwd, vwd, W, o_w, lse_w)
    torch.cuda.synchronize()
    assert torch.isneginf(lse_sp).all()
    dq = torch.empty(B, L, Hq, D, **f32)
    dk, dv = torch.full((B, L, Hkv, D), 3.0, **f32), torch.full((B, L, Hkv, D), 3.0, **f32)
    dkw, dvw = torch.empty(B, L, Hkv, D, **f32), torch.empty(B, L, Hkv, D, **f32)
    dgw = torch.empty(Hq, D, **f32)
    ops.hys_sparse_layer_bwd(qd, kd, vd, idx, kwd, vwd, W, gw.to(dev), o_sp, lse_sp, o_w, lse_w, do.to(dev), dq, dk,
                             dv, dkw, dvw, dgw, accumulate_kv=True, topk=0)
    torch.cuda.synchronize()
    none = np.full((L, 1), -1)
    r = hb.sparse_layer_bwd(_f64(q[0]), _f64(k[0]), _f64(v[0]), _f64(kw[0]), _f64(vw[0]),
                            gw.numpy().astype(np.float64), scale, none, 64, W, _f64(do[0]))
    assert not r["dk"].any() and not r["dgate_w"].any()
    assert torch.equal(dk, torch.full_like(dk, 3.0)) and torch.equal(dv, torch.full_like(dv, 3.0))
    assert not dgw.any()
    check_grad(dq[0].cpu().numpy(), r["dq"], "dq (window only)")
    check_grad(dkw[0].cpu().numpy(), r["dkw"], "dk_win (window only)")
    check_grad(dvw[0].cpu().numpy(), r["dvw"], "dv_win (window only)")
