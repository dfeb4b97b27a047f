"""GPU parity at the five workloads' full sizes, in the launch configuration
bench.py times (the block runners of hybrid_sparse_attention_flash_amd.block).

The whole hybrid block runs on the GPU; the oracle recomputes sampled query
rows (or sampled 64-query tiles, or every decode sequence) one by one from the
same seeded inputs and the outputs are compared with the rules of
tests/parity_util.py.  Sparse-layer outputs are compared on every sampled row:
where the GPU's top-k differs from the oracle's inside the tie band (both are
correct), the oracle is re-evaluated on the GPU's selection
(parity_util.selection_to_compare), and each test asserts how many rows and
layers it compared.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from hybrid_sparse_attention_flash_amd.block import HySparse2Block, HySparse2Decode, HySparseBlock
from tests.parity_util import TOL_OUT, check_out, check_scores, check_topk_band, max_abs, selection_to_compare

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


def _hysparse_case(name, nrows, seed=0, out_dtype=torch.float32):
    w = synth.WORKLOADS[name]
    print(f"workload {name}: generating inputs (outputs {out_dtype})", flush=True)
    q = [synth.gen_q(w, l, seed) for l in range(w.n_sparse + 1)]
    k, _ = synth.gen_kv(w, "k", seed)
    v, _ = synth.gen_kv(w, "v", seed)
    kw = [synth.gen_window_kv(w, l + 1, "kw", seed)[0] for l in range(w.n_sparse)]
    vw = [synth.gen_window_kv(w, l + 1, "vw", seed)[0] for l in range(w.n_sparse)]
    gw = [synth.gen_gate_w(w, l + 1, seed) for l in range(w.n_sparse)]
    blk = HySparseBlock(w.B, w.L, w.Hq, w.Hkv, w.D, w.n_sparse, w.topk, w.window, device="cuda",
                        out_dtype=out_dtype)
    print(f"workload {name}: running the block on the GPU", flush=True)
    blk.run([x.cuda() for x in q], k.cuda(), v.cuda(), [x.cuda() for x in kw], [x.cuda() for x in vw],
            [x.cuda() for x in gw])
    torch.cuda.synchronize()
    rows = _sample_rows(w.L, nrows, extra=(63, 64, 65, 127, 128, w.L - 64, w.L - 63))
    print(f"workload {name}: oracle on {len(rows)} rows", flush=True)
    f = lambda t: t[0].to(torch.float64).numpy()
    kf, vf = f(k), f(v)
    qv = [RowView(x[0]) for x in q]
    gw64 = [x.numpy().astype(np.float64) for x in gw]
    ref = oracle.hysparse_block(qv, kf, vf, [f(x) for x in kw], [f(x) for x in vw], gw64, w.scale, w.block,
                                w.topk, w.window, rows=rows)
    tol = TOL_OUT[w.q_dtype]
    r = torch.as_tensor(rows)
    check_out(blk.o_full[0][r].float().cpu().numpy(), ref["o_full"], w.q_dtype, "o_full")
    assert max_abs(blk.lse[0][:, r].cpu().numpy(), ref["lse"]) <= max(tol, 1e-3)
    check_scores(blk.scores[0, 0][r].cpu().numpy(), ref["scores"])
    gidx = blk.idx[0, 0][r].cpu().numpy()
    same, inband = check_topk_band(gidx, ref["sel"], ref["scores"], w.topk)
    print(f"workload {name}: top-k rows identical {same}, inside the tie band {inband}", flush=True)
    # rows whose GPU selection differs inside the band: the oracle's sparse
    # layers re-evaluated on the GPU's selection
    diff = [i for i in range(len(rows))
            if not selection_to_compare(gidx[i], ref["sel"][i], ref["scores"][i], w.topk)[1]]
    compared = 0
    for l in range(w.n_sparse):
        want = np.array(ref["o_layers"][l])
        if diff:
            rd = rows[diff]
            o_sp, lse_sp = oracle.sparse_block_attention(qv[l + 1], kf, vf, w.scale, gidx[diff], w.block, rd)
            o_w, _ = oracle.window_attention(qv[l + 1], f(kw[l]), f(vw[l]), w.scale, w.window, rd)
            want[diff] = oracle.gate_merge(qv[l + 1][rd], gw64[l], o_sp, lse_sp, o_w)
        got = blk.o_layers[l][0][r].float().cpu().numpy()
        check_out(got, want, w.q_dtype, f"sparse layer {l}")
        compared += len(rows)
    print(f"workload {name}: sparse layers compared on {compared} (row, layer) pairs, "
          f"{len(diff)} rows on the GPU's in-band selection", flush=True)
    assert compared == w.n_sparse * len(rows)


def test_tiny_fp32_whole_block():
    """The tiny fp32 workload (L=1024) is compared on every row."""
    _hysparse_case("tiny_fp32", 1024)


def test_dense7b_16k_sampled_rows():
    _hysparse_case("dense7b_16k", 24)


def test_moe80b_32k_sampled_rows():
    _hysparse_case("moe80b_32k", 16)


def test_moe80b_32k_bf16_outputs_bench_configuration():
    """The 32k block exactly as bench.py times it: bf16 outputs, so the
    one-pass sparse layer's bf16 epilogue is checked at full size."""
    _hysparse_case("moe80b_32k", 24, out_dtype=torch.bfloat16)


@pytest.mark.timeout(600)
def test_hysparse2_64k_sampled_tiles():
    """Eight query tiles spread over the 64k sequence, every one past 1024
    visible keys (so each has a non-trivial top-1024).  Each tile's token
    scores and top-k are checked whole; the full layer and all three sparse
    layers on eight rows of the tile (its first and last row among them).
    The oracle is composed from its pinned parts exactly as
    oracle.hysparse2_block composes them, evaluated on those rows only."""
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
    ntile = w.L // w.block
    first = w.topk // w.block + 1            # tile 17 sees 1088 keys
    tiles = np.unique(np.linspace(first, ntile - 1, 8).round().astype(np.int64))
    assert len(tiles) == 8 and tiles[0] * w.block + 1 > w.topk
    kf = oracle.as_f64(k[0], "fp8", ks)
    vf = oracle.as_f64(v[0], "fp8", vs)
    qv = [RowView(x[0]) for x in q]
    compared = moved = 0
    for t in tiles:
        print(f"workload hysparse2_64k: oracle on tile {t}", flush=True)
        T = oracle.tile_token_scores(qv[0], kf, w.scale, w.block, [t])
        check_scores(blk.scores[0][t:t + 1].cpu().numpy(), T)
        sel_ref, _ = oracle.topk_rows(T, w.topk)
        gidx = blk.idx[0][t:t + 1].cpu().numpy()
        check_topk_band(gidx, sel_ref, T, w.topk)
        sel, same = selection_to_compare(gidx[0], sel_ref[0], T[0], w.topk)
        moved += 0 if same else 1
        rows = t * w.block + np.array([0, 9, 18, 27, 36, 45, 54, 63])
        rr = torch.as_tensor(rows)
        o_full, _ = oracle.full_attention(qv[0], kf, vf, w.scale, rows)
        check_out(blk.o_full[0][rr].cpu().numpy(), o_full, "bf16", f"tile {t} o_full")
        sel_tiles = np.full((ntile, w.topk), -1, dtype=np.int64)
        sel_tiles[t] = sel
        for l in range(w.n_sparse):
            want, _ = oracle.sparse_token_attention(qv[l + 1], kf, vf, w.scale, sel_tiles, w.block, w.window, rows)
            check_out(blk.o_layers[l][0][rr].cpu().numpy(), want, "bf16", f"tile {t} layer {l}")
            compared += 1
    print(f"workload hysparse2_64k: tiles {tiles.tolist()}, {compared} (tile, layer) comparisons, "
          f"{moved} tiles on the GPU's in-band selection", flush=True)
    assert compared == len(tiles) * w.n_sparse


# Ragged valid lengths inside the 1,048,576-token caches (the bench times the
# workload with every cache full): a full cache, one token short, a length
# that ends inside a 64-key tile and half a cache plus a partial tile.
DECODE_1M_RAGGED = (1048576, 1048575, 786433, 524353)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("lens", [None, DECODE_1M_RAGGED], ids=["full_caches", "ragged"])
def test_decode_1m_all_sequences(lens):
    w = synth.WORKLOADS["decode_1m"]
    if lens is not None:
        w = w.shrink(cache_lens=lens)
    print(f"workload decode_1m: generating inputs, lengths {w.lens()}", flush=True)
    qf = synth.gen_q(w, 0)
    qs = [synth.gen_q(w, l + 1) for l in range(w.n_sparse)]
    kc, ks = synth.gen_kv(w, "k")
    vc, vs = synth.gen_kv(w, "v")
    dec = HySparse2Decode(w.B, w.L, w.Hq, w.D, w.n_sparse, w.topk, w.window, device="cuda")
    print("workload decode_1m: running the decode step on the GPU", flush=True)
    dec.run(qf.cuda(), kc.cuda(), vc.cuda(), w.lens(), [x.cuda() for x in qs], ks, vs)
    torch.cuda.synchronize()
    compared = 0
    for b in range(w.B):
        n = w.lens()[b]
        print(f"workload decode_1m: oracle on sequence {b} (n = {n})", flush=True)
        kf = oracle.as_f64(kc[b], "fp8", ks)
        vf = oracle.as_f64(vc[b], "fp8", vs)
        qs_b = [x[b, 0].to(torch.float64).numpy() for x in qs]
        res = oracle.decode_step(qf[b, 0].to(torch.float64).numpy(), kf, vf, w.scale, n, qs_b, w.topk, w.window)
        check_out(dec.o_full[b, 0].cpu().numpy(), res["o_full"], "bf16", "o_full")
        s = dec.scores[b].cpu().numpy()
        check_scores(s[:n], res["scores"])
        assert np.all(np.isneginf(s[n:]))
        gi = dec.idx[b].cpu().numpy()
        check_topk_band(gi[None], res["sel"][None], res["scores"][None], w.topk)
        sel, same = selection_to_compare(gi, res["sel"], res["scores"], w.topk)
        for l in range(w.n_sparse):
            want = res["o_layers"][l] if same else oracle.decode_sparse(qs_b[l], kf, vf, w.scale, n, sel, w.window)[0]
            check_out(dec.o_layers[l][b, 0].cpu().numpy(), want, "bf16", f"sequence {b} sparse layer {l}")
            compared += 1
        del kf, vf
    assert compared == w.B * w.n_sparse
