"""The seeded input generator: determinism, independence and storage conversions."""
import hashlib

import numpy as np
import torch

import synth


def _sha(t):
    return hashlib.sha256(t.contiguous().view(torch.uint8).numpy().tobytes()).hexdigest()


def test_deterministic_and_independent():
    w = synth.WORKLOADS["tiny_fp32"]
    a = synth.gen_q(w, 1, seed=0)
    b = synth.gen_q(w, 1, seed=0)
    c = synth.gen_q(w, 2, seed=0)
    d = synth.gen_q(w, 1, seed=1)
    assert _sha(a) == _sha(b)
    assert _sha(a) != _sha(c) and _sha(a) != _sha(d)
    assert a.shape == (1, 1024, 8, 64) and a.dtype == torch.float32


def test_bf16_round_to_nearest_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -8 + 2 ** -20, -2.5], np.float32)
    y = synth.to_bf16(x).to(torch.float64).numpy()
    # ties go to the even mantissa: 1+2^-8 -> 1, 1+3*2^-8 -> 1+2^-6; above a tie rounds up
    np.testing.assert_array_equal(y, [1.0, 1.0, 1.0 + 2 ** -6, 1.0 + 2 ** -7, -2.5])


def test_fp8_scale_and_range():
    x = synth.normal(0, 9, "t", (4096,))
    codes, s = synth.to_fp8_e4m3(x)
    vals = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy() * s
    assert abs(np.abs(vals).max() - np.abs(x).max()) <= np.abs(x).max() * 2 ** -4
    assert np.abs(vals - x).max() <= np.abs(x).max() * 2 ** -4
    assert not np.isnan(vals).any()


def test_needles_scale_k_only():
    w = synth.WORKLOADS["moe80b_32k"].shrink(L=512, Hq=4, Hkv=1, needles=8)
    pos = synth.needle_positions(w)
    assert len(pos) == 8 and len(set(pos.tolist())) == 8 and pos.max() < 512
    k, _ = synth.gen_kv(w, "k")
    w0 = w.shrink(needles=0)
    k0, _ = synth.gen_kv(w0, "k")
    ratio = (k.float()[0, pos] / k0.float()[0, pos]).flatten()
    finite = torch.isfinite(ratio) & (k0.float()[0, pos].flatten().abs() > 0.05)
    assert torch.allclose(ratio[finite], torch.tensor(4.0), rtol=2e-2)
    mask = torch.ones(512, dtype=torch.bool)
    mask[pos] = False
    assert torch.equal(k[0, mask], k0[0, mask])
    v, _ = synth.gen_kv(w, "v")
    v0, _ = synth.gen_kv(w0, "v")
    assert torch.equal(v, v0)


def test_workload_table():
    ws = synth.WORKLOADS
    assert [ws[n].cfg_id for n in synth.WORKLOAD_ORDER] == [1, 2, 3, 4, 5]
    assert ws["moe80b_32k"].n_sparse == 11 and ws["dense7b_16k"].n_sparse == 3
    assert ws["hysparse2_64k"].topk == 1024 and ws["hysparse2_64k"].Hkv == 1
    assert ws["decode_1m"].L == 1 << 20 and ws["decode_1m"].B == 4
