"""GPU parity at the five workloads' full sizes, in the launch configuration
bench.py times (the block runners of hybrid_sparse_attention_flash_amd.block).

The whole hybrid block runs on the GPU; the oracle recomputes sampled query
rows (or sampled 64-query tiles, or every decode sequence) one by one from the
same seeded inputs and the outputs are compared with the rules of
tests/parity_util.py.  Sparse-layer outputs are compared on the rows whose
selected index sets are identical on both sides (rows inside the top-k tie
band select differently by construction).
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from hybrid_sparse_attention_flash_amd.block import HySparse2Block, HySparse2Decode, HySparseBlock
from tests.parity_util import TOL_OUT, check_out, check_scores, check_topk_band, max_abs

pytestmark = pytest.mark.gpu


class RowView:
    """Float64 view of a stored [L, H, D] tensor that converts only indexed rows."""

    def __init__(self, t):
        self.t = t
        self.shape = tuple(t.shape)

    def __getitem__(self, rows):
        return self.t[torch.as_tensor(np.asarray(rows))].to(torch.float64).numpy()


def _sample_rows(L, n, extra=()):
    rows = set(np.linspace(0, L - 1, n).round().astype(int).tolist())
    rows |= {r for r in extra if 0 <= r < L}
    return np.array(sorted(rows), dtype=np.int64)


def _hysparse_case(name, nrows, seed=0):
    w = synth.WORKLOADS[name]
    print(f"workload {name}: generating inputs", flush=True)
    q = [synth.gen_q(w, l, seed) for l in range(w.n_sparse + 1)]
    k, _ = synth.gen_kv(w, "k", seed)
    v, _ = synth.gen_kv(w, "v", seed)
    kw = [synth.gen_window_kv(w, l + 1, "kw", seed)[0] for l in range(w.n_sparse)]
    vw = [synth.gen_window_kv(w, l + 1, "vw", seed)[0] for l in range(w.n_sparse)]
    gw = [synth.gen_gate_w(w, l + 1, seed) for l in range(w.n_sparse)]
    blk = HySparseBlock(w.B, w.L, w.Hq, w.Hkv, w.D, w.n_sparse, w.topk, w.window, device="cuda",
                        out_dtype=torch.float32)
    print(f"workload {name}: running the block on the GPU", flush=True)
    blk.run([x.cuda() for x in q], k.cuda(), v.cuda(), [x.cuda() for x in kw], [x.cuda() for x in vw],
            [x.cuda() for x in gw])
    torch.cuda.synchronize()
    rows = _sample_rows(w.L, nrows, extra=(63, 64, 65, 127, 128, w.L - 64, w.L - 63))
    print(f"workload {name}: oracle on {len(rows)} rows", flush=True)
    f = lambda t: t[0].to(torch.float64).numpy()
    ref = oracle.hysparse_block([RowView(x[0]) for x in q], f(k), f(v), [f(x) for x in kw], [f(x) for x in vw],
                                [x.numpy().astype(np.float64) for x in gw], w.scale, w.block, w.topk, w.window,
                                rows=rows)
    tol = TOL_OUT[w.q_dtype]
    r = torch.as_tensor(rows)
    check_out(blk.o_full[0][r].cpu().numpy(), ref["o_full"], w.q_dtype, "o_full")
    assert max_abs(blk.lse[0][:, r].cpu().numpy(), ref["lse"]) <= max(tol, 1e-3)
    check_scores(blk.scores[0, 0][r].cpu().numpy(), ref["scores"])
    gidx = blk.idx[0, 0][r].cpu().numpy()
    same, inband = check_topk_band(gidx, ref["sel"], ref["scores"], w.topk)
    eq = np.array([np.array_equal(gidx[i], ref["sel"][i]) for i in range(len(rows))])
    print(f"workload {name}: top-k rows identical {same}, inside the tie band {inband}", flush=True)
    assert eq.sum() >= len(rows) - 2
    for l in range(w.n_sparse):
        got = blk.o_layers[l][0][r].cpu().numpy()
        check_out(got[eq], ref["o_layers"][l][eq], w.q_dtype, f"sparse layer {l}")


def test_tiny_fp32_whole_block():
    """The tiny fp32 workload (L=1024) is compared on every row."""
    _hysparse_case("tiny_fp32", 1024)


def test_dense7b_16k_sampled_rows():
    _hysparse_case("dense7b_16k", 24)


def test_moe80b_32k_sampled_rows():
    _hysparse_case("moe80b_32k", 16)


def test_hysparse2_64k_sampled_tiles():
    w = synth.WORKLOADS["hysparse2_64k"]
    print("workload hysparse2_64k: generating inputs", flush=True)
    q = [synth.gen_q(w, l) for l in range(w.n_sparse + 1)]
    k, ks = synth.gen_kv(w, "k")
    v, vs = synth.gen_kv(w, "v")
    blk = HySparse2Block(w.B, w.L, w.Hq, w.Hkv, w.D, w.n_sparse, w.topk, w.window, tile=w.block, device="cuda",
                         out_dtype=torch.float32)
    print("workload hysparse2_64k: running the block on the GPU", flush=True)
    blk.run([x.cuda() for x in q], k.cuda(), v.cuda(), ks, vs)
    torch.cuda.synchronize()
    tiles = np.array([3, w.L // 64 - 1])
    print(f"workload hysparse2_64k: oracle on tiles {tiles.tolist()}", flush=True)
    kf = oracle.as_f64(k[0], "fp8", ks)
    vf = oracle.as_f64(v[0], "fp8", vs)
    ref = oracle.hysparse2_block([RowView(x[0]) for x in q], kf, vf, w.scale, w.block, w.topk, w.window, tiles=tiles)
    rows = torch.as_tensor(ref["rows"])
    check_out(blk.o_full[0][rows].cpu().numpy(), ref["o_full"], "bf16", "o_full")
    check_scores(blk.scores[0][torch.as_tensor(tiles)].cpu().numpy(), ref["scores"])
    gidx = blk.idx[0][torch.as_tensor(tiles)].cpu().numpy()
    same, inband = check_topk_band(gidx, ref["sel"], ref["scores"], w.topk)
    print(f"workload hysparse2_64k: top-k tiles identical {same}, inside the tie band {inband}", flush=True)
    for n, t in enumerate(tiles):
        if not np.array_equal(gidx[n], ref["sel"][n]):
            continue
        sl = slice(n * 64, (n + 1) * 64)
        for l in range(w.n_sparse):
            got = blk.o_layers[l][0][rows[sl]].cpu().numpy()
            check_out(got, ref["o_layers"][l][sl], "bf16", f"tile {t} layer {l}")


def test_decode_1m_all_sequences():
    w = synth.WORKLOADS["decode_1m"]
    print("workload decode_1m: generating inputs", flush=True)
    qf = synth.gen_q(w, 0)
    qs = [synth.gen_q(w, l + 1) for l in range(w.n_sparse)]
    kc, ks = synth.gen_kv(w, "k")
    vc, vs = synth.gen_kv(w, "v")
    dec = HySparse2Decode(w.B, w.L, w.Hq, w.D, w.n_sparse, w.topk, w.window, device="cuda")
    print("workload decode_1m: running the decode step on the GPU", flush=True)
    dec.run(qf.cuda(), kc.cuda(), vc.cuda(), w.lens(), [x.cuda() for x in qs], ks, vs)
    torch.cuda.synchronize()
    for b in range(w.B):
        n = w.lens()[b]
        print(f"workload decode_1m: oracle on sequence {b}", flush=True)
        kf = oracle.as_f64(kc[b], "fp8", ks)
        vf = oracle.as_f64(vc[b], "fp8", vs)
        res = oracle.decode_step(qf[b, 0].to(torch.float64).numpy(), kf, vf, w.scale, n,
                                 [x[b, 0].to(torch.float64).numpy() for x in qs], w.topk, w.window)
        del kf, vf
        check_out(dec.o_full[b, 0].cpu().numpy(), res["o_full"], "bf16", "o_full")
        check_scores(dec.scores[b].cpu().numpy()[:n], res["scores"])
        gi = dec.idx[b].cpu().numpy()
        same, inband = check_topk_band(gi[None], res["sel"][None], res["scores"][None], w.topk)
        if same:
            for l in range(w.n_sparse):
                check_out(dec.o_layers[l][b, 0].cpu().numpy(), res["o_layers"][l], "bf16", "o_sparse")
