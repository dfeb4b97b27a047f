"""GPU parity of the ablation variants against the oracle.

  * per-KV-group selection: per-group block scores (HYS_SCORE_BLOCK_GROUP),
    top-k over every group's rows, the block-sparse branch and the fused
    sparse layer with per-group index sets, and the whole HySparse block;
  * HySparse2 with a gated window branch over the shared fp8 cache instead
    of the forced window;
  * block-level selection at the token budget (hys_select_topk_blocks) and
    the HySparse2 block run with it.
Selections are compared bit-exact with the oracle's selection taken on the
GPU's own fp32 scores (the integer decision on the same values); outputs by
the rules of tests/parity_util.py, computed by the oracle with the GPU's
selection.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from hybrid_sparse_attention_flash_amd import ops
from hybrid_sparse_attention_flash_amd.block import HySparse2Block, HySparseBlock
from tests.parity_util import check_out, check_scores

pytestmark = pytest.mark.gpu


def _hs_inputs(name, seed=0, **kw):
    w = synth.WORKLOADS[name].shrink(**kw)
    q = [synth.gen_q(w, l, seed) for l in range(w.n_sparse + 1)]
    k, ks = synth.gen_kv(w, "k", seed)
    v, vs = synth.gen_kv(w, "v", seed)
    return w, q, k, ks, v, vs


@pytest.mark.parametrize("name,L,Hq,Hkv,D", [("dense7b_16k", 300, 8, 4, 128), ("tiny_fp32", 200, 8, 2, 64)])
def test_per_group_scores_and_grouped_sparse(name, L, Hq, Hkv, D):
    w, q, k, ks, v, vs = _hs_inputs(name, L=L, Hq=Hq, Hkv=Hkv, D=D, n_sparse=1, topk=3)
    dt = w.q_dtype
    nblk = (L + 63) // 64
    qd, kd, vd = q[0].cuda(), k.cuda(), v.cuda()
    o = torch.empty(1, L, Hq, D, dtype=torch.float32, device="cuda")
    sc = torch.empty(Hkv, 1, L, nblk, dtype=torch.float32, device="cuda")
    ops.hys_full_attn_fwd(qd, kd, vd, o, None, "block_group", sc)
    torch.cuda.synchronize()
    f = lambda t: oracle.as_f64(t[0], dt)
    Mg = oracle.block_scores_per_group(f(q[0]), f(k), w.scale, 64)
    for g in range(Hkv):
        check_scores(sc[g, 0].cpu().numpy(), Mg[g])
    # top-k over every group's rows; the oracle selects on the GPU's scores
    idx = torch.empty(Hkv, 1, L, w.topk, dtype=torch.int32, device="cuda")
    ops.hys_select_topk(sc.view(Hkv * L, nblk), w.topk, idx.view(Hkv * L, w.topk))
    torch.cuda.synchronize()
    sel_ref, _ = oracle.topk_rows(sc.view(Hkv * L, nblk).cpu().numpy().astype(np.float64), w.topk)
    assert np.array_equal(idx.view(Hkv * L, w.topk).cpu().numpy(), sel_ref)
    sel_g = idx[:, 0].cpu().numpy()
    # block-sparse branch with per-group index sets
    o_sp = torch.empty(1, L, Hq, D, dtype=torch.float32, device="cuda")
    lse_sp = torch.empty(1, Hq, L, dtype=torch.float32, device="cuda")
    ops.hys_sparse_attn_fwd(q[1].cuda(), kd, vd, idx, o_sp, lse_sp, granularity=64, topk=w.topk)
    torch.cuda.synchronize()
    O, LSE = oracle.sparse_block_attention_grouped(f(q[1]), f(k), f(v), w.scale, sel_g, 64)
    check_out(o_sp[0].cpu().numpy(), O, dt, "grouped sparse o")
    fin = np.isfinite(LSE)
    assert np.array_equal(np.isfinite(lse_sp[0].cpu().numpy()), fin)
    assert np.max(np.abs(lse_sp[0].cpu().numpy()[fin] - LSE[fin])) <= 1e-3
    # fused sparse layer (grouped sparse + own window + gate) with per-group sets
    kw, _ = synth.gen_window_kv(w, 1, "kw")
    vw, _ = synth.gen_window_kv(w, 1, "vw")
    gw = synth.gen_gate_w(w, 1)
    o_l = torch.empty(1, L, Hq, D, dtype=torch.float32, device="cuda")
    ops.hys_sparse_layer_fwd(q[1].cuda(), kd, vd, idx, kw.cuda(), vw.cuda(), w.window, gw.cuda(), o_l, topk=w.topk)
    torch.cuda.synchronize()
    o_w, _ = oracle.window_attention(f(q[1]), f(kw), f(vw), w.scale, w.window)
    ref = oracle.gate_merge(f(q[1]), gw.numpy().astype(np.float64), O, LSE, o_w)
    check_out(o_l[0].cpu().numpy(), ref, dt, "fused grouped sparse layer")


def test_hysparse_block_kv_group_selection():
    w, q, k, _, v, _ = _hs_inputs("moe80b_32k", L=320, Hq=16, Hkv=4, D=128, n_sparse=2, topk=3,
                                     needles=4)
    kw = [synth.gen_window_kv(w, l, "kw")[0] for l in range(1, 3)]
    vw = [synth.gen_window_kv(w, l, "vw")[0] for l in range(1, 3)]
    gw = [synth.gen_gate_w(w, l) for l in range(1, 3)]
    blk = HySparseBlock(w.B, w.L, w.Hq, w.Hkv, w.D, 2, w.topk, w.window, device="cuda", selection="kv_group")
    blk.run([x.cuda() for x in q], k.cuda(), v.cuda(), [x.cuda() for x in kw], [x.cuda() for x in vw],
            [x.cuda() for x in gw])
    torch.cuda.synchronize()
    f = lambda t: oracle.as_f64(t[0], "bf16")
    Mg = oracle.block_scores_per_group(f(q[0]), f(k), w.scale, 64)
    for g in range(w.Hkv):
        check_scores(blk.scores[g, 0].cpu().numpy(), Mg[g])
    rows = w.Hkv * w.L
    sel_ref, _ = oracle.topk_rows(blk.scores.view(rows, -1).cpu().numpy().astype(np.float64), w.topk)
    assert np.array_equal(blk.idx.view(rows, -1).cpu().numpy(), sel_ref)
    sel_g = blk.idx[:, 0].cpu().numpy()
    for l in range(2):
        O, LSE = oracle.sparse_block_attention_grouped(f(q[l + 1]), f(k), f(v), w.scale, sel_g, 64)
        o_w, _ = oracle.window_attention(f(q[l + 1]), f(kw[l]), f(vw[l]), w.scale, w.window)
        ref = oracle.gate_merge(f(q[l + 1]), gw[l].numpy().astype(np.float64), O, LSE, o_w)
        check_out(blk.o_layers[l][0].cpu().numpy(), ref, "bf16", f"layer {l}")


def _hs2_case(window_mode, selection, L=330, seed=0):
    w, q, k, ks, v, vs = _hs_inputs("hysparse2_64k", seed=seed, L=L, Hq=8, n_sparse=2, topk=256)
    gw = [synth.gen_gate_w(w, l) for l in range(1, 3)]
    blk = HySparse2Block(w.B, w.L, w.Hq, w.Hkv, w.D, 2, w.topk, w.window, tile=64, device="cuda",
                         window_mode=window_mode, selection=selection)
    blk.run([x.cuda() for x in q], k.cuda(), v.cuda(), ks, vs, gate_layers=[x.cuda() for x in gw])
    torch.cuda.synchronize()
    f = lambda t: oracle.as_f64(t[0], "bf16")
    kf, vf = oracle.as_f64(k[0], "fp8", ks), oracle.as_f64(v[0], "fp8", vs)
    return w, q, gw, blk, f, kf, vf


def test_hysparse2_gated_window():
    w, q, gw, blk, f, kf, vf = _hs2_case("gated", "token")
    T = oracle.tile_token_scores(f(q[0]), kf, w.scale, 64)
    check_scores(blk.scores[0].cpu().numpy(), T)
    sel = blk.idx[0].cpu().numpy()
    sel_ref, _ = oracle.topk_rows(blk.scores[0].cpu().numpy().astype(np.float64), w.topk)
    assert np.array_equal(sel, sel_ref)
    for l in range(2):
        ref = oracle.hysparse2_gated_window_layer(f(q[l + 1]), kf, vf, w.scale, sel, 64, w.window,
                                                  gw[l].numpy().astype(np.float64))
        check_out(blk.o_layers[l][0].cpu().numpy(), ref, "bf16", f"gated layer {l}")


def test_select_topk_blocks_rows():
    g = torch.Generator().manual_seed(7)
    rows, cols, kb = 37, 1000, 3
    x = torch.randn(rows, cols, generator=g)
    x[5, 700:] = float("-inf")                        # a row whose tail is not visible
    x[6] = float("-inf")
    x[6, 10] = 1.0                                    # one visible block only
    x[9, 195] = 11.0                                  # block 3 first, then blocks 0, 1, 2 tied:
    x[9, 3] = x[9, 67] = x[9, 131] = 10.0             # the lowest ids win the tie
    xd = x.cuda()
    idx = torch.empty(rows, 64 * kb, dtype=torch.int32, device="cuda")
    ops.hys_select_topk_blocks(xd, kb, idx)
    torch.cuda.synchronize()
    Mt = oracle.tile_block_scores(x.numpy().astype(np.float64), 64)
    sel, _ = oracle.topk_rows(Mt, kb)
    ref = oracle.expand_blocks(sel, 64, cols)
    assert np.array_equal(idx.cpu().numpy(), ref)


def test_hysparse2_block_level_selection_at_token_budget():
    w, q, gw, blk, f, kf, vf = _hs2_case("forced", "block")
    T = oracle.tile_token_scores(f(q[0]), kf, w.scale, 64)
    check_scores(blk.scores[0].cpu().numpy(), T)
    Mt = oracle.tile_block_scores(blk.scores[0].cpu().numpy().astype(np.float64), 64)
    selb, _ = oracle.topk_rows(Mt, w.topk // 64)
    sel_ref = oracle.expand_blocks(selb, 64, w.L)
    sel = blk.idx[0].cpu().numpy()
    assert np.array_equal(sel, sel_ref)
    for l in range(2):
        ref, _ = oracle.sparse_token_attention(f(q[l + 1]), kf, vf, w.scale, sel, 64, w.window)
        check_out(blk.o_layers[l][0].cpu().numpy(), ref, "bf16", f"block-level layer {l}")
