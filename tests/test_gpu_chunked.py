"""GPU parity of chunked prefill: a call whose queries are rows
[q_offset, q_offset + Lq) of a longer sequence, attending to the cache of all
Lk >= q_offset + Lq keys (hys_attn_params.q_offset).

The oracle evaluates the whole sequence's definitions at the chunk's absolute
rows (oracle functions take `rows`), so the check is the plain statement that
a chunk computes exactly what the whole sequence computes at those rows:
the full layer with block or tile-token scores, the selection, and the sparse
layers (HySparse one-pass and two-call forms, HySparse2 token-sparse) for
offsets that cut tiles and blocks and for chunks that end before the cache.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from hybrid_sparse_attention_flash_amd import ops
from tests.parity_util import TOL_OUT, check_out, check_scores, check_topk_band, f64, max_abs, selection_to_compare

pytestmark = pytest.mark.gpu


def _nan(shape, dtype=torch.float32):
    return torch.full(shape, float("nan"), dtype=dtype, device="cuda")


@pytest.mark.parametrize("name,L,Hq,Hkv,D,q_off,Lq", [
    ("tiny_fp32", 300, 4, 1, 64, 100, 150),     # chunk inside the cache, offset cutting a block
    ("tiny_fp32", 300, 4, 2, 64, 237, 63),      # chunk ending at the cache end
    ("dense7b_16k", 400, 8, 2, 128, 64, 300),   # block-aligned offset
    ("dense7b_16k", 400, 8, 2, 128, 1, 399),
    ("moe80b_32k", 520, 16, 2, 128, 333, 120),
])
def test_chunked_hysparse_block(name, L, Hq, Hkv, D, q_off, Lq):
    w = synth.WORKLOADS[name].shrink(L=L, Hq=Hq, Hkv=Hkv, D=D, n_sparse=1, topk=4,
                                     needles=4 if name == "moe80b_32k" else 0)
    qa = synth.gen_q(w, 0)
    q1 = synth.gen_q(w, 1)
    k, _ = synth.gen_kv(w, "k")
    v, _ = synth.gen_kv(w, "v")
    kw, _ = synth.gen_window_kv(w, 1, "kw")
    vw, _ = synth.gen_window_kv(w, 1, "vw")
    gw = synth.gen_gate_w(w, 1)
    W = 128
    print(f"chunked hysparse {name} L={L} Hq={Hq} Hkv={Hkv} D={D} q_offset={q_off} Lq={Lq}", flush=True)
    sl = slice(q_off, q_off + Lq)
    qc, q1c = qa[:, sl].contiguous().cuda(), q1[:, sl].contiguous().cuda()
    kd, vd, kwd, vwd = k.cuda(), v.cuda(), kw.cuda(), vw.cuda()
    nblk = (L + 63) // 64
    o = _nan((1, Lq, Hq, D))
    lse = _nan((1, Hq, Lq))
    sc = _nan((1, Lq, nblk))
    ops.hys_full_attn_fwd(qc, kd, vd, o, lse, "block", sc, q_offset=q_off)
    idx = torch.full((1, Lq, w.topk), -7, dtype=torch.int32, device="cuda")
    ops.hys_select_topk(sc.view(Lq, nblk), w.topk, idx.view(Lq, w.topk))
    o1 = _nan((1, Lq, Hq, D))
    ops.hys_sparse_layer_fwd(q1c, kd, vd, idx, kwd, vwd, W, gw.cuda(), o1, q_offset=q_off)
    # the two-call form of the same layer
    osp = _nan((1, Lq, Hq, D))
    lsp = _nan((1, Hq, Lq))
    ops.hys_sparse_attn_fwd(q1c, kd, vd, idx, osp, lsp, granularity=64, q_offset=q_off)
    o2 = _nan((1, Lq, Hq, D))
    ops.hys_swa_gate_fwd(q1c, kwd, vwd, W, osp, lsp, gw.cuda(), o2, q_offset=q_off)
    torch.cuda.synchronize()

    rows = np.arange(q_off, q_off + Lq)
    qf, q1f = f64(qa[0], w.q_dtype), f64(q1[0], w.q_dtype)
    kf, vf = f64(k[0], w.kv_dtype), f64(v[0], w.kv_dtype)
    O, LSE = oracle.full_attention(qf, kf, vf, w.scale, rows)
    M = oracle.block_scores(qf, kf, w.scale, 64, rows)
    check_out(o[0].cpu().numpy(), O, w.q_dtype, "o_full")
    assert max_abs(lse[0].cpu().numpy(), LSE) <= max(TOL_OUT[w.q_dtype], 1e-3)
    check_scores(sc[0].cpu().numpy(), M)
    sel_ref, _ = oracle.topk_rows(M, w.topk)
    gi = idx[0].cpu().numpy()
    check_topk_band(gi, sel_ref, M, w.topk)
    sel = np.stack([selection_to_compare(gi[r], sel_ref[r], M[r], w.topk)[0] for r in range(Lq)])
    o_sp, lse_sp = oracle.sparse_block_attention(q1f, kf, vf, w.scale, sel, 64, rows)
    o_w, _ = oracle.window_attention(q1f, f64(kw[0], w.q_dtype), f64(vw[0], w.q_dtype), w.scale, W, rows)
    want = oracle.gate_merge(q1f[rows], gw.numpy().astype(np.float64), o_sp, lse_sp, o_w)
    check_out(o1[0].cpu().numpy(), want, w.q_dtype, "one-pass sparse layer")
    check_out(osp[0].cpu().numpy(), o_sp, w.q_dtype, "sparse branch")
    check_out(o2[0].cpu().numpy(), want, w.q_dtype, "two-call sparse layer")


@pytest.mark.parametrize("L,Hq,D,q_off,Lq,topk", [
    (400, 8, 128, 128, 272, 100),     # to the end of the cache, ragged last tile
    (300, 4, 64, 64, 236, 50),
    (700, 8, 128, 512, 128, 256),     # two whole tiles inside the cache
])
def test_chunked_hysparse2_tiles(L, Hq, D, q_off, Lq, topk):
    """HySparse2 chunks start on a 64-query tile (the selection is per tile)
    and end on a tile boundary or at the cache end, so each of the chunk's
    tiles is a tile of the whole sequence."""
    w = synth.WORKLOADS["hysparse2_64k"].shrink(L=L, Hq=Hq, D=D, n_sparse=1, topk=topk)
    qa = synth.gen_q(w, 0)
    q1 = synth.gen_q(w, 1)
    k, ks = synth.gen_kv(w, "k")
    v, vs = synth.gen_kv(w, "v")
    W = 128
    print(f"chunked hysparse2 L={L} Hq={Hq} D={D} q_offset={q_off} Lq={Lq} topk={topk}", flush=True)
    sl = slice(q_off, q_off + Lq)
    qc, q1c = qa[:, sl].contiguous().cuda(), q1[:, sl].contiguous().cuda()
    kd, vd = k.cuda(), v.cuda()
    nt = (Lq + 63) // 64
    o = _nan((1, Lq, Hq, D))
    sc = _nan((1, nt, L))
    ops.hys_full_attn_fwd(qc, kd, vd, o, None, "tile_token", sc, k_scale=ks, v_scale=vs, q_offset=q_off)
    idx = torch.full((1, nt, topk), -7, dtype=torch.int32, device="cuda")
    ops.hys_select_topk(sc.view(nt, L), topk, idx.view(nt, topk))
    o1 = _nan((1, Lq, Hq, D))
    ops.hys_sparse_attn_fwd(q1c, kd, vd, idx, o1, None, granularity=1, q_tile=64, forced_window=W, k_scale=ks,
                            v_scale=vs, q_offset=q_off)
    torch.cuda.synchronize()

    rows = np.arange(q_off, q_off + Lq)
    tiles = q_off // 64 + np.arange(nt)
    qf, q1f = f64(qa[0]), f64(q1[0])
    kf, vf = oracle.as_f64(k[0], "fp8", ks), oracle.as_f64(v[0], "fp8", vs)
    O, _ = oracle.full_attention(qf, kf, vf, w.scale, rows)
    check_out(o[0].cpu().numpy(), O, "bf16", "o_full")
    T = oracle.tile_token_scores(qf, kf, w.scale, 64, tiles)
    check_scores(sc[0].cpu().numpy(), T)
    sel_ref, _ = oracle.topk_rows(T, topk)
    gi = idx[0].cpu().numpy()
    check_topk_band(gi, sel_ref, T, topk)
    sel_tiles = np.full(((L + 63) // 64, topk), -1, dtype=np.int64)
    for n, t in enumerate(tiles):
        sel_tiles[t] = selection_to_compare(gi[n], sel_ref[n], T[n], topk)[0]
    want, _ = oracle.sparse_token_attention(q1f, kf, vf, w.scale, sel_tiles, 64, W, rows)
    check_out(o1[0].cpu().numpy(), want, "bf16", "token-sparse layer")
