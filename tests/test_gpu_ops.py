"""GPU parity of each C-ABI call against the fp64 oracle, on small seeded inputs.

Shapes span several 64-key tiles and end on ragged tails; every call goes
through the C ABI (libhys.so) via the ctypes binding.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import synth
from hybrid_sparse_attention_flash_amd import ops
from tests.parity_util import (TOL_OUT, check_out, check_scores, check_topk_band, dev, f64, max_abs,
                               selection_to_compare)

pytestmark = pytest.mark.gpu


def _wl(name, **kw):
    return synth.WORKLOADS[name].shrink(**kw)


def _qkv(w, seed=0):
    q = synth.gen_q(w, 0, seed)
    k, ks = synth.gen_kv(w, "k", seed)
    v, vs = synth.gen_kv(w, "v", seed)
    return q, k, ks, v, vs


def _nan_like(shape, dtype=torch.float32):
    return torch.full(shape, float("nan"), dtype=dtype, device="cuda")


FULL_CASES = [
    # name, L, Hq, Hkv, D, q dtype (kv dtype follows the workload)
    ("tiny_fp32", 1024, 8, 1, 64),
    ("tiny_fp32", 130, 4, 2, 64),
    ("tiny_fp32", 65, 2, 1, 128),
    ("dense7b_16k", 200, 8, 2, 128),
    ("dense7b_16k", 129, 4, 4, 64),
    ("dense7b_16k", 1, 4, 1, 128),
    ("moe80b_32k", 320, 16, 2, 128),
]


@pytest.mark.parametrize("name,L,Hq,Hkv,D", FULL_CASES)
def test_full_attention_block_scores(name, L, Hq, Hkv, D):
    w = _wl(name, L=L, Hq=Hq, Hkv=Hkv, D=D, needles=min(4, L) if name == "moe80b_32k" else 0)
    q, k, ks, v, vs = _qkv(w)
    print(f"full+block {name} L={L} Hq={Hq} Hkv={Hkv} D={D}", flush=True)
    o = _nan_like((w.B, L, Hq, D))
    lse = _nan_like((w.B, Hq, L))
    nblk = (L + 63) // 64
    sc = _nan_like((w.B, L, nblk))
    ops.hys_full_attn_fwd(dev(q), dev(k), dev(v), o, lse, "block", sc)
    torch.cuda.synchronize()
    tol = TOL_OUT[w.q_dtype]
    for b in range(w.B):
        qf, kf, vf = f64(q[b], w.q_dtype), f64(k[b], w.kv_dtype), f64(v[b], w.kv_dtype)
        O, LSE = oracle.full_attention(qf, kf, vf, w.scale)
        M = oracle.block_scores(qf, kf, w.scale, 64)
        check_out(o[b].cpu().numpy(), O, w.q_dtype, "o")
        assert max_abs(lse[b].cpu().numpy(), LSE) <= max(tol, 1e-3)
        check_scores(sc[b].cpu().numpy(), M)


# Head groupings of the bf16 full layer: the query's heads reduced for the
# block score across 2..32 adjacent lanes, a query spanning several waves
# (G = 64), groups that do not divide 32 (G = 6: the heads of a query straddle
# two waves), no scores, and bf16 outputs.
FULL_GROUP_CASES = [
    # L, Hq, Hkv, D, score mode, output dtype
    (300, 16, 1, 128, "block", torch.float32),
    (133, 32, 1, 128, "block", torch.bfloat16),
    (200, 4, 2, 64, "block", torch.bfloat16),
    (150, 6, 1, 128, "block", torch.float32),
    (257, 8, 1, 128, "none", torch.bfloat16),
    (97, 64, 1, 64, "none", torch.float32),
    (64, 8, 2, 128, "block", torch.bfloat16),
]


@pytest.mark.parametrize("L,Hq,Hkv,D,mode,odt", FULL_GROUP_CASES)
def test_full_attention_head_groups(L, Hq, Hkv, D, mode, odt):
    w = _wl("dense7b_16k", L=L, Hq=Hq, Hkv=Hkv, D=D)
    q, k, ks, v, vs = _qkv(w, seed=L + Hq)
    print(f"full {mode} L={L} Hq={Hq} Hkv={Hkv} D={D} out={odt}", flush=True)
    o = _nan_like((w.B, L, Hq, D), odt)
    lse = _nan_like((w.B, Hq, L))
    nblk = (L + 63) // 64
    sc = _nan_like((w.B, L, nblk)) if mode == "block" else None
    ops.hys_full_attn_fwd(dev(q), dev(k), dev(v), o, lse, mode, sc)
    torch.cuda.synchronize()
    for b in range(w.B):
        qf, kf, vf = f64(q[b], w.q_dtype), f64(k[b], w.kv_dtype), f64(v[b], w.kv_dtype)
        O, LSE = oracle.full_attention(qf, kf, vf, w.scale)
        check_out(o[b].float().cpu().numpy(), O, "bf16", "o")
        assert max_abs(lse[b].cpu().numpy(), LSE) <= 1e-3
        if mode == "block":
            check_scores(sc[b].cpu().numpy(), oracle.block_scores(qf, kf, w.scale, 64))


TILE_CASES = [
    ("hysparse2_64k", 300, 8, 1, 128),
    ("hysparse2_64k", 128, 4, 1, 64),
    ("dense7b_16k", 190, 8, 2, 128),
]


@pytest.mark.parametrize("name,L,Hq,Hkv,D", TILE_CASES)
def test_full_attention_tile_token_scores(name, L, Hq, Hkv, D):
    w = _wl(name, L=L, Hq=Hq, Hkv=Hkv, D=D)
    q, k, ks, v, vs = _qkv(w)
    print(f"full+tile {name} L={L} Hq={Hq} Hkv={Hkv} D={D} kv={w.kv_dtype}", flush=True)
    o = _nan_like((1, L, Hq, D))
    lse = _nan_like((1, Hq, L))
    nt = (L + 63) // 64
    sc = _nan_like((1, nt, L))
    ops.hys_full_attn_fwd(dev(q), dev(k), dev(v), o, lse, "tile_token", sc, k_scale=ks, v_scale=vs)
    torch.cuda.synchronize()
    qf, kf, vf = f64(q[0]), oracle.as_f64(k[0], w.kv_dtype, ks), oracle.as_f64(v[0], w.kv_dtype, vs)
    O, LSE = oracle.full_attention(qf, kf, vf, w.scale)
    T = oracle.tile_token_scores(qf, kf, w.scale, 64)
    check_out(o[0].cpu().numpy(), O, "bf16", "o")
    assert max_abs(lse[0].cpu().numpy(), LSE) <= 1e-3
    check_scores(sc[0].cpu().numpy(), T)


@pytest.mark.parametrize("rows,cols,k", [(300, 16, 4), (257, 512, 16), (64, 2048, 64), (33, 3000, 100),
                                         (5, 65536, 1024), (3, 200001, 1024), (4, 32768, 1000), (2, 1048576, 1024),
                                         (2, 1048576 + 4096, 1024), (1, 3000001, 2048),
                                         (7, 100, 0), (9, 40, 50), (6, 2048, 16), (6, 1000, 65), (5, 64, 64),
                                         (8, 700, 33)])
def test_select_topk_exact(rows, cols, k):
    """Same fp32 scores on both sides -> the index sets must be identical."""
    r = np.random.default_rng(rows * 7 + cols)
    x = np.round(r.standard_normal((rows, cols)), 2).astype(np.float32)   # many exact ties
    x[r.random((rows, cols)) < 0.05] = -np.inf
    x[r.random((rows, cols)) < 0.01] = np.nan
    if rows > 2:
        x[1, :] = -np.inf                       # a row with no candidate
        x[2, : cols // 2] = -np.inf             # causal-like row
    if rows > 3:
        x[3, :] = 0.5                           # one value everywhere: every candidate ties
    if rows > 4:
        x[4, :] = -1.0
        x[4, 1::2] = -0.0                       # -0 and +0 are equal scores: they tie, the lower column wins
        x[4, ::4] = 0.0
    print(f"topk rows={rows} cols={cols} k={k}", flush=True)
    s = torch.from_numpy(x).cuda()
    idx = torch.full((rows, max(k, 1)), -7, dtype=torch.int32, device="cuda")[:, :k].contiguous()
    cnt = torch.full((rows,), -7, dtype=torch.int32, device="cuda")
    ops.hys_select_topk(s, k, idx, cnt)
    torch.cuda.synchronize()
    gi, gc = idx.cpu().numpy(), cnt.cpu().numpy()
    for row in range(rows):
        ref, rc = oracle.topk_select(x[row].astype(np.float64), k)
        assert gi[row].tolist() == ref.tolist(), (row, gi[row][:8], ref[:8])
        assert gc[row] == rc


def _rand_block_sel(L, k, rng):
    sel = np.full((L, k), -1, dtype=np.int32)
    for i in range(L):
        nb = i // 64 + 1
        c = np.sort(rng.choice(nb, size=min(k, nb), replace=False))
        if rng.random() < 0.1:
            c = c[: max(0, len(c) - 1)]         # fewer than k valid
        sel[i, :len(c)] = c
    return sel


@pytest.mark.parametrize("name,L,Hq,Hkv,D,k", [("tiny_fp32", 1024, 8, 1, 64, 4), ("dense7b_16k", 333, 8, 2, 128, 3),
                                               ("moe80b_32k", 512, 16, 2, 128, 6), ("dense7b_16k", 200, 4, 4, 64, 0)])
def test_sparse_block_attention(name, L, Hq, Hkv, D, k):
    w = _wl(name, L=L, Hq=Hq, Hkv=Hkv, D=D, needles=0)
    q = synth.gen_q(w, 1)
    kk, _ = synth.gen_kv(w, "k")
    vv, _ = synth.gen_kv(w, "v")
    sel = _rand_block_sel(L, k, np.random.default_rng(L))
    print(f"sparse-block {name} L={L} Hq={Hq} Hkv={Hkv} D={D} k={k}", flush=True)
    o = _nan_like((1, L, Hq, D))
    lse = _nan_like((1, Hq, L))
    idx = torch.from_numpy(sel).reshape(1, L, k).cuda() if k > 0 else torch.zeros((1, L, 1), dtype=torch.int32,
                                                                                  device="cuda")
    ops.hys_sparse_attn_fwd(dev(q), dev(kk), dev(vv), idx, o, lse, granularity=64, topk=k, q_tile=1)
    torch.cuda.synchronize()
    O, LSE = oracle.sparse_block_attention(f64(q[0], w.q_dtype), f64(kk[0], w.kv_dtype), f64(vv[0], w.kv_dtype),
                                           w.scale, sel if k > 0 else np.zeros((L, 0), int), 64)
    check_out(o[0].cpu().numpy(), O, w.q_dtype, "o")
    g = lse[0].cpu().numpy()
    assert np.array_equal(np.isneginf(g), np.isneginf(LSE))
    fin = np.isfinite(LSE)
    assert max_abs(g[fin], LSE[fin]) <= 1e-3


@pytest.mark.parametrize("L,Hq,D,k,W,kv", [(300, 8, 128, 40, 16, "fp8"), (640, 4, 128, 100, 128, "fp8"),
                                           (200, 8, 64, 0, 128, "bf16"), (129, 2, 128, 3000 // 30, 8, "fp8")])
def test_sparse_token_attention(L, Hq, D, k, W, kv):
    w = _wl("hysparse2_64k", L=L, Hq=Hq, D=D, kv_dtype=kv)
    q = synth.gen_q(w, 1)
    kk, ks = synth.gen_kv(w, "k")
    vv, vs = synth.gen_kv(w, "v")
    nt = (L + 63) // 64
    rng = np.random.default_rng(L + k)
    sel = np.full((nt, max(k, 1)), -1, dtype=np.int32)
    for t in range(nt):
        hi = min(L, (t + 1) * 64)
        c = np.sort(rng.choice(hi, size=min(k, hi), replace=False))
        sel[t, :len(c)] = c
    sel = sel[:, :k] if k > 0 else sel[:, :0]
    print(f"sparse-token L={L} Hq={Hq} D={D} k={k} W={W} kv={kv}", flush=True)
    o = _nan_like((1, L, Hq, D))
    lse = _nan_like((1, Hq, L))
    idx = torch.from_numpy(np.ascontiguousarray(sel)).reshape(1, nt, k).cuda() if k > 0 else \
        torch.zeros((1, nt, 1), dtype=torch.int32, device="cuda")
    ops.hys_sparse_attn_fwd(dev(q), dev(kk), dev(vv), idx, o, lse, granularity=1, topk=k, q_tile=64,
                            forced_window=W, k_scale=ks, v_scale=vs)
    torch.cuda.synchronize()
    O, LSE = oracle.sparse_token_attention(f64(q[0]), oracle.as_f64(kk[0], kv, ks), oracle.as_f64(vv[0], kv, vs),
                                           w.scale, sel, 64, W)
    check_out(o[0].cpu().numpy(), O, "bf16", "o")
    assert max_abs(lse[0].cpu().numpy(), LSE) <= 1e-3


@pytest.mark.parametrize("name,L,Hq,Hkv,D,W", [("tiny_fp32", 1024, 8, 1, 64, 128), ("dense7b_16k", 300, 8, 2, 128, 128),
                                               ("dense7b_16k", 100, 4, 1, 64, 1), ("moe80b_32k", 200, 8, 8, 128, 77)])
def test_swa_gate(name, L, Hq, Hkv, D, W):
    w = _wl(name, L=L, Hq=Hq, Hkv=Hkv, D=D, needles=0)
    q = synth.gen_q(w, 1)
    kw, _ = synth.gen_window_kv(w, 1, "kw")
    vw, _ = synth.gen_window_kv(w, 1, "vw")
    gw = synth.gen_gate_w(w, 1)
    r = np.random.default_rng(L)
    o_sp = r.standard_normal((1, L, Hq, D)).astype(np.float32)
    lse_sp = r.standard_normal((1, Hq, L)).astype(np.float32)
    lse_sp[0, :, ::7] = -np.inf                      # empty sparse sets on some rows
    print(f"swa-gate {name} L={L} Hq={Hq} Hkv={Hkv} D={D} W={W}", flush=True)
    o = _nan_like((1, L, Hq, D))
    ops.hys_swa_gate_fwd(dev(q), dev(kw), dev(vw), W, torch.from_numpy(o_sp).cuda(), torch.from_numpy(lse_sp).cuda(),
                         dev(gw), o)
    torch.cuda.synchronize()
    qf = f64(q[0], w.q_dtype)
    Ow, _ = oracle.window_attention(qf, f64(kw[0], w.q_dtype), f64(vw[0], w.q_dtype), w.scale, W)
    ref = oracle.gate_merge(qf, gw.numpy().astype(np.float64), o_sp[0].astype(np.float64),
                            lse_sp[0].astype(np.float64), Ow)
    check_out(o[0].cpu().numpy(), ref, w.q_dtype, "o")


@pytest.mark.parametrize("name,L,Hq,Hkv,D,k,W,out", [
    ("tiny_fp32", 1024, 8, 1, 64, 4, 128, "f32"),
    ("dense7b_16k", 333, 8, 2, 128, 3, 128, "f32"),
    ("moe80b_32k", 512, 16, 2, 128, 6, 77, "f32"),
    ("moe80b_32k", 300, 8, 1, 128, 16, 128, "bf16"),
    ("dense7b_16k", 200, 4, 4, 64, 0, 1, "f32"),
    # 16-row-block kernel (bf16, 2..16 heads per KV head): every head ratio,
    # both head dims, an empty selection, ragged lengths
    ("dense7b_16k", 200, 8, 4, 64, 0, 1, "f32"),
    ("moe80b_32k", 150, 32, 2, 128, 5, 128, "bf16"),
    ("moe80b_32k", 333, 16, 2, 64, 8, 100, "f32"),
    ("dense7b_16k", 257, 16, 4, 128, 2, 40, "bf16"),
])
def test_sparse_layer_fused(name, L, Hq, Hkv, D, k, W, out):
    """The one-pass sparse layer against the oracle's sparse branch, window branch and gate."""
    w = _wl(name, L=L, Hq=Hq, Hkv=Hkv, D=D, needles=0)
    q = synth.gen_q(w, 1)
    kk, _ = synth.gen_kv(w, "k")
    vv, _ = synth.gen_kv(w, "v")
    kw, _ = synth.gen_window_kv(w, 1, "kw")
    vw, _ = synth.gen_window_kv(w, 1, "vw")
    gw = synth.gen_gate_w(w, 1)
    sel = _rand_block_sel(L, k, np.random.default_rng(L + 7))
    if k > 0:
        sel[::9] = -1                                  # rows with an empty selection
    print(f"sparse-layer {name} L={L} Hq={Hq} Hkv={Hkv} D={D} k={k} W={W} out={out}", flush=True)
    odt = torch.float32 if out == "f32" else torch.bfloat16
    o = _nan_like((1, L, Hq, D), odt)
    idx = torch.from_numpy(sel).reshape(1, L, k).cuda() if k > 0 else torch.zeros((1, L, 1), dtype=torch.int32,
                                                                                  device="cuda")
    ops.hys_sparse_layer_fwd(dev(q), dev(kk), dev(vv), idx, dev(kw), dev(vw), W, dev(gw), o, topk=k)
    torch.cuda.synchronize()
    qf = f64(q[0], w.q_dtype)
    Osp, LSEsp = oracle.sparse_block_attention(qf, f64(kk[0], w.kv_dtype), f64(vv[0], w.kv_dtype), w.scale,
                                               sel if k > 0 else np.zeros((L, 0), int), 64)
    Ow, _ = oracle.window_attention(qf, f64(kw[0], w.q_dtype), f64(vw[0], w.q_dtype), w.scale, W)
    ref = oracle.gate_merge(qf, gw.numpy().astype(np.float64), Osp, LSEsp, Ow)
    got = o[0].float().cpu().numpy()
    assert np.isfinite(got).all()
    check_out(got, ref, w.q_dtype if out == "f32" else "bf16", "o")


@pytest.mark.parametrize("B,N,lens,Hq,D,topk,W,nsp,kv", [
    (2, 5000, (5000, 3001), 64, 128, 256, 128, 3, "fp8"),
    (3, 700, (1, 64, 700), 16, 128, 64, 32, 2, "fp8"),
    (1, 70000, (69999,), 64, 128, 1024, 128, 1, "fp8"),
    (2, 900, (900, 513), 8, 64, 100, 16, 2, "bf16"),
])
def test_decode_step(B, N, lens, Hq, D, topk, W, nsp, kv):
    w = _wl("decode_1m", B=B, L=N, Hq=Hq, D=D, kv_dtype=kv, n_sparse=nsp, topk=topk, window=W, cache_lens=lens)
    qf = synth.gen_q(w, 0)
    qs = [synth.gen_q(w, l + 1) for l in range(nsp)]
    kc, ks = synth.gen_kv(w, "k")
    vc, vs = synth.gen_kv(w, "v")
    print(f"decode B={B} N={N} lens={lens} Hq={Hq} D={D} topk={topk} W={W} nsp={nsp} kv={kv}", flush=True)
    o_full = _nan_like((B, 1, Hq, D))
    scores = _nan_like((B, N))
    idx = torch.full((B, topk), -7, dtype=torch.int32, device="cuda")
    o_sp = [_nan_like((B, 1, Hq, D)) for _ in range(nsp)]
    ops.hys_decode_step(dev(qf), dev(kc), dev(vc), list(lens), o_full, scores, idx, [dev(x) for x in qs], o_sp,
                        topk, W, k_scale=ks, v_scale=vs)
    torch.cuda.synchronize()
    compared = 0
    for b in range(B):
        n = lens[b]
        kf = oracle.as_f64(kc[b, :, 0:1], kv, ks)
        vf = oracle.as_f64(vc[b, :, 0:1], kv, vs)
        res = oracle.decode_step(f64(qf[b, 0]), kf, vf, w.scale, n, [f64(x[b, 0]) for x in qs], topk, W)
        check_out(o_full[b, 0].cpu().numpy(), res["o_full"], "bf16", "o_full")
        s = scores[b].cpu().numpy()
        check_scores(s[:n], res["scores"])
        assert np.all(np.isneginf(s[n:]))
        gi = idx[b].cpu().numpy()
        check_topk_band(gi[None], res["sel"][None], res["scores"][None], topk)
        # every sparse layer is compared: on the oracle's selection, or on the
        # GPU's where it differs inside the tie band
        sel, same = selection_to_compare(gi, res["sel"], res["scores"], topk)
        for l in range(nsp):
            want = res["o_layers"][l] if same else oracle.decode_sparse(f64(qs[l][b, 0]), kf, vf, w.scale, n, sel, W)[0]
            check_out(o_sp[l][b, 0].cpu().numpy(), want, "bf16", f"o_sparse layer {l}")
            compared += 1
    assert compared == B * nsp


@pytest.mark.parametrize("half", [0, 1])
def test_fp8_codec_exact(half):
    """Every finite e4m3fn code decodes exactly on the HIP path.

    With one token the softmax weight is exactly 1, so the full layer's output
    row is the dequantised V row: O[0,h,d] = decode(byte_d) * v_scale, bit for bit
    (fp32 output; decoding to bf16 is exact for every finite e4m3 value).
    """
    codes = np.arange(128, dtype=np.uint8) + np.uint8(128 * half)
    codes[codes == 0x7F] = 0x00
    codes[codes == 0xFF] = 0x80
    vscale = 0.375
    q = torch.zeros((1, 1, 4, 128), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((1, 1, 1, 128), dtype=torch.uint8, device="cuda")
    v = torch.from_numpy(codes).reshape(1, 1, 1, 128).cuda()
    o = _nan_like((1, 1, 4, 128))
    ops.hys_full_attn_fwd(q, k, v, o, None, "none", None, k_scale=1.0, v_scale=vscale)
    torch.cuda.synchronize()
    want = oracle.fp8.dequantize(codes, vscale)
    got = o[0, 0].cpu().numpy().astype(np.float64)
    for h in range(4):
        np.testing.assert_array_equal(got[h], want)
