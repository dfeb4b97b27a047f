"""GPU parity of the ablation variants at the full workload sizes, in the
launch configurations bench.py times with --selection / --window-mode.

The oracle recomputes sampled query rows (HySparse, 32k) or sampled 64-query
tiles (HySparse2, 64k) from the same seeded inputs.  Scores are compared
directly; selections are compared with the top-k tie band of
tests/parity_util.py, and outputs on the rows whose selections are identical
(rows inside the band select differently by construction).
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from hybrid_sparse_attention_flash_amd.block import HySparse2Block, HySparseBlock
from tests.parity_util import check_out, check_scores, check_topk_band, selection_to_compare

pytestmark = pytest.mark.gpu


class RowView:
    """Float64 view of a stored [L, H, D] tensor that converts only indexed rows."""

    def __init__(self, t):
        self.t = t
        self.shape = tuple(t.shape)

    def __getitem__(self, rows):
        return self.t[torch.as_tensor(np.asarray(rows))].to(torch.float64).numpy()


def test_moe80b_32k_kv_group_selection_sampled_rows():
    w = synth.WORKLOADS["moe80b_32k"]
    print("kv_group 32k: generating inputs", flush=True)
    q = [synth.gen_q(w, l) for l in range(w.n_sparse + 1)]
    k, v = synth.gen_kv(w, "k")[0], synth.gen_kv(w, "v")[0]
    kw = [synth.gen_window_kv(w, l + 1, "kw")[0] for l in range(w.n_sparse)]
    vw = [synth.gen_window_kv(w, l + 1, "vw")[0] for l in range(w.n_sparse)]
    gw = [synth.gen_gate_w(w, l + 1) for l in range(w.n_sparse)]
    blk = HySparseBlock(w.B, w.L, w.Hq, w.Hkv, w.D, w.n_sparse, w.topk, w.window, device="cuda",
                        out_dtype=torch.float32, selection="kv_group")
    print("kv_group 32k: running the block on the GPU", flush=True)
    blk.run([x.cuda() for x in q], k.cuda(), v.cuda(), [x.cuda() for x in kw], [x.cuda() for x in vw],
            [x.cuda() for x in gw])
    torch.cuda.synchronize()
    rows = np.array(sorted(set(np.linspace(0, w.L - 1, 12).round().astype(int).tolist()) | {63, 64, w.L - 1}))
    r = torch.as_tensor(rows)
    kf, vf = k[0].to(torch.float64).numpy(), v[0].to(torch.float64).numpy()
    print(f"kv_group 32k: oracle on {len(rows)} rows", flush=True)
    Mg = oracle.block_scores_per_group(RowView(q[0][0]), kf, w.scale, 64, rows)
    sel_g = np.stack([oracle.topk_rows(Mg[g], w.topk)[0] for g in range(w.Hkv)])
    # the selection every sparse layer is compared on: the oracle's, or the
    # GPU's where it differs inside the tie band (both correct)
    sel_use = np.empty_like(sel_g)
    for g in range(w.Hkv):
        check_scores(blk.scores[g, 0][r].cpu().numpy(), Mg[g])
        gi = blk.idx[g, 0][r].cpu().numpy()
        same, inband = check_topk_band(gi, sel_g[g], Mg[g], w.topk)
        print(f"kv_group 32k: group {g} top-k rows identical {same}, inside the tie band {inband}", flush=True)
        for i in range(len(rows)):
            sel_use[g][i] = selection_to_compare(gi[i], sel_g[g][i], Mg[g][i], w.topk)[0]
    compared = 0
    for l in range(w.n_sparse):
        ql = RowView(q[l + 1][0])
        O, LSE = oracle.sparse_block_attention_grouped(ql, kf, vf, w.scale, sel_use, 64, rows)
        o_w, _ = oracle.window_attention(ql, kw[l][0].to(torch.float64).numpy(), vw[l][0].to(torch.float64).numpy(),
                                         w.scale, w.window, rows)
        ref = oracle.gate_merge(ql[rows], gw[l].numpy().astype(np.float64), O, LSE, o_w)
        check_out(blk.o_layers[l][0][r].cpu().numpy(), ref, "bf16", f"kv_group layer {l}")
        compared += 1
    assert compared == w.n_sparse


@pytest.mark.timeout(600)
def test_hysparse2_64k_gated_window_and_block_selection_sampled_tiles():
    w = synth.WORKLOADS["hysparse2_64k"]
    print("hysparse2 variants 64k: generating inputs", flush=True)
    q = [synth.gen_q(w, l) for l in range(w.n_sparse + 1)]
    k, ks = synth.gen_kv(w, "k")
    v, vs = synth.gen_kv(w, "v")
    gw = [synth.gen_gate_w(w, l + 1) for l in range(w.n_sparse)]
    qd, kd, vd = [x.cuda() for x in q], k.cuda(), v.cuda()
    gated = HySparse2Block(w.B, w.L, w.Hq, w.Hkv, w.D, w.n_sparse, w.topk, w.window, tile=w.block, device="cuda",
                           out_dtype=torch.float32, window_mode="gated")
    blocks = HySparse2Block(w.B, w.L, w.Hq, w.Hkv, w.D, w.n_sparse, w.topk, w.window, tile=w.block, device="cuda",
                            out_dtype=torch.float32, selection="block")
    print("hysparse2 variants 64k: running both blocks on the GPU", flush=True)
    gated.run(qd, kd, vd, ks, vs, gate_layers=[x.cuda() for x in gw])
    blocks.run(qd, kd, vd, ks, vs)
    torch.cuda.synchronize()
    del qd
    ntile = w.L // 64
    tiles = np.array([17, 512, ntile - 1])    # each sees more than 1024 keys
    kf, vf = oracle.as_f64(k[0], "fp8", ks), oracle.as_f64(v[0], "fp8", vs)
    print(f"hysparse2 variants 64k: oracle on tiles {tiles.tolist()}", flush=True)
    T = oracle.tile_token_scores(RowView(q[0][0]), kf, w.scale, 64, tiles)
    tt = torch.as_tensor(tiles)
    check_scores(gated.scores[0][tt].cpu().numpy(), T)
    check_scores(blocks.scores[0][tt].cpu().numpy(), T)
    # gated window: token selection as the default block, then the gated layer
    sel_t, _ = oracle.topk_rows(T, w.topk)
    gi = gated.idx[0][tt].cpu().numpy()
    check_topk_band(gi, sel_t, T, w.topk)
    sel_full = np.full((ntile, w.topk), -1, dtype=np.int64)
    for n, t in enumerate(tiles):
        sel_full[t] = selection_to_compare(gi[n], sel_t[n], T[n], w.topk)[0]
    # block selection at the token budget: top topk/64 blocks of the tile rows,
    # expanded; the GPU's chosen blocks are read back from its expanded rows
    kb = w.topk // 64
    Mt = oracle.tile_block_scores(T, 64)
    selb, _ = oracle.topk_rows(Mt, kb)
    bi = blocks.idx[0][tt].cpu().numpy()
    sel_bfull = np.full((ntile, w.topk), -1, dtype=np.int64)
    for n, t in enumerate(tiles):
        gb = np.unique(bi[n][bi[n] >= 0] // 64)
        gb = np.concatenate([gb, np.full(kb - len(gb), -1)]).astype(np.int64)
        use, _ = selection_to_compare(gb, selb[n], Mt[n], kb)
        expanded = oracle.expand_blocks(use[None], 64, w.L)[0]
        assert np.array_equal(bi[n], expanded), f"tile {t}: expansion of the GPU's blocks"
        sel_bfull[t] = expanded
    compared = 0
    for n, t in enumerate(tiles):
        rows = t * 64 + np.array([0, 21, 42, 63])
        rr = torch.as_tensor(rows)
        for l in range(w.n_sparse):
            ql = RowView(q[l + 1][0])
            ref = oracle.hysparse2_gated_window_layer(ql, kf, vf, w.scale, sel_full, 64, w.window,
                                                      gw[l].numpy().astype(np.float64), rows)
            check_out(gated.o_layers[l][0][rr].cpu().numpy(), ref, "bf16", f"gated tile {t} layer {l}")
            ref, _ = oracle.sparse_token_attention(ql, kf, vf, w.scale, sel_bfull, 64, w.window, rows)
            check_out(blocks.o_layers[l][0][rr].cpu().numpy(), ref, "bf16", f"block-level tile {t} layer {l}")
            compared += 2
    print(f"hysparse2 variants 64k: gated selections identical {[np.array_equal(gi[i], sel_t[i]) for i in range(3)]}, "
          f"{compared} comparisons", flush=True)
    assert compared == 2 * len(tiles) * w.n_sparse
