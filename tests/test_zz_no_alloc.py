"""hys_decode_step_noalloc (the decode step on the library's fixed scratch
array, for callers that cannot allocate) against hys_decode_step with a
caller-provided workspace, through the C ABI.

Two calls in a row on the same GPU, the second smaller than the first, so
the second runs on scratch that still holds the first call's values: every
output must equal the workspace entry point's bit for bit (same kernels,
deterministic merge and selection), with outputs poisoned with NaN before
each call so that anything left unwritten shows.
"""
import numpy as np
import pytest
import torch

import synth
from hybrid_sparse_attention_flash_amd import ops

pytestmark = pytest.mark.gpu


def _nan(shape):
    return torch.full(shape, float("nan"), dtype=torch.float32, device="cuda")


def _run_both(B, N, lens, Hq, D, topk, W, nsp):
    w = synth.WORKLOADS["decode_1m"].shrink(B=B, L=N, Hq=Hq, D=D, n_sparse=nsp, topk=topk, window=W,
                                             cache_lens=tuple(lens))
    qf = synth.gen_q(w, 0).cuda()
    qs = [synth.gen_q(w, l + 1).cuda() for l in range(nsp)]
    kc, ks = synth.gen_kv(w, "k")
    vc, vs = synth.gen_kv(w, "v")
    kc, vc = kc.cuda(), vc.cuda()
    print(f"no-alloc decode B={B} N={N} lens={lens} Hq={Hq} D={D} topk={topk} W={W} nsp={nsp}", flush=True)
    out = {}
    for name in ("workspace", "noalloc"):
        o_full = _nan((B, 1, Hq, D))
        scores = _nan((B, N))
        idx = torch.full((B, topk), -7, dtype=torch.int32, device="cuda")
        o_sp = [_nan((B, 1, Hq, D)) for _ in range(nsp)]
        fn = ops.hys_decode_step if name == "workspace" else ops.hys_decode_step_noalloc
        fn(qf, kc, vc, list(lens), o_full, scores, idx, qs, o_sp, topk, W, k_scale=ks, v_scale=vs)
        torch.cuda.synchronize()
        out[name] = (o_full.cpu(), scores.cpu(), idx.cpu(), [x.cpu() for x in o_sp])
    a, b = out["workspace"], out["noalloc"]
    assert torch.isfinite(b[0]).all()
    assert torch.equal(a[0], b[0]), "o_full differs"
    assert torch.equal(a[1], b[1]), "token scores differ"
    assert torch.equal(a[2], b[2]), "selection differs"
    for l in range(nsp):
        assert torch.isfinite(b[3][l]).all()
        assert torch.equal(a[3][l], b[3][l]), f"sparse layer {l} differs"
    return b


def test_noalloc_decode_matches_workspace_entry_point_twice():
    first = _run_both(4, 300000, (300000, 299999, 150001, 70000), 64, 128, 1024, 128, 3)
    second = _run_both(2, 5000, (5000, 3001), 64, 128, 256, 128, 2)
    assert second[2].shape == (2, 256) and first[2].shape == (4, 1024)
    assert (second[2][1] >= 0).sum().item() == 256
