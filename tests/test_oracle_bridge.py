"""Pins of the KV Bridging oracle (projection + fp8 e4m3 quantisation).

The encoder is checked against torch's CPU float8_e4m3fn conversion (an
independent implementation of the same format) over dense value sets and every
rounding midpoint, against the decode table (round trip of all finite codes),
and on the saturation and NaN readings; the projection against pure-Python
loops; the precision rule on a value that the fp32 rounding moves onto a
midpoint.  A dropped scale, a wrong tie rule, an off-by-one exponent at a
power of two or a transposed weight fails one of them.
"""
import numpy as np
import torch

from oracle.bridge import encode_e4m3, kv_bridge, quantize_kernel_precision
from oracle.fp8 import decode_table

TAB = decode_table()
FINITE = np.array([b for b in range(256) if not np.isnan(TAB[b])], dtype=np.int64)


def _torch_codes(x32: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(x32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_encoder_round_trips_every_finite_code():
    assert np.array_equal(encode_e4m3(TAB[FINITE]), FINITE.astype(np.uint8))


def test_encoder_matches_torch_in_range():
    rng = np.random.default_rng(3)
    x = np.concatenate([rng.standard_normal(20000).astype(np.float32) * s for s in (1e-3, 0.03, 1.0, 40.0, 180.0)])
    x = x[np.abs(x) < 464.0]
    vals = np.sort(TAB[FINITE])
    mids = ((vals[:-1] + vals[1:]) / 2).astype(np.float32)
    # one fp32 ulp on either side of every midpoint
    up = np.nextafter(mids, np.float32(np.inf))
    dn = np.nextafter(mids, np.float32(-np.inf))
    allx = np.concatenate([x, mids, up, dn, -mids, np.float32([0.0, -0.0, 448.0, -448.0, 464.0, -464.0])])
    allx = allx[np.abs(allx) <= 464.0].astype(np.float32)
    assert np.array_equal(encode_e4m3(allx.astype(np.float64)), _torch_codes(allx))


def test_encoder_saturation_and_nan():
    # torch (non-saturating) turns these into NaN; the cache reading saturates
    assert encode_e4m3(np.array([480.0, 500.0, 1e30, -1e30])).tolist() == [0x7E, 0x7E, 0x7E, 0xFE]
    assert encode_e4m3(np.array([np.nan])).tolist() == [0x7F]
    assert encode_e4m3(np.array([2.0 ** -10, 3 * 2.0 ** -11, 15 * 2.0 ** -10])).tolist() == [0x00, 0x01, 0x08]


def test_kv_bridge_brute_force():
    rng = np.random.default_rng(11)
    B, L, d, N = 2, 3, 5, 4
    h = rng.standard_normal((B, L, d))
    wk = rng.standard_normal((N, d))
    wv = rng.standard_normal((N, d))
    ks, vs = 0.013, 0.021
    kc, vc, kx, vx, ak, av = kv_bridge(h, wk, wv, ks, vs)
    inv_k = np.float32(1.0) / np.float32(ks)
    inv_v = np.float32(1.0) / np.float32(vs)
    for b in range(B):
        for t in range(L):
            for n in range(N):
                sk = sum(h[b, t, c] * wk[n, c] for c in range(d))
                sv = sum(h[b, t, c] * wv[n, c] for c in range(d))
                assert abs(kx[b, t, n] - sk) < 1e-12 and abs(vx[b, t, n] - sv) < 1e-12
                assert kc[b, t, n] == _torch_codes(np.array([np.float32(sk) * inv_k]))[0] \
                    or abs(float(np.float32(sk) * inv_k)) > 448
                assert vc[b, t, n] == _torch_codes(np.array([np.float32(sv) * inv_v]))[0] \
                    or abs(float(np.float32(sv) * inv_v)) > 448
    assert ak == max(abs(x) for x in kx.ravel()) and av == max(abs(x) for x in vx.ravel())


def test_kv_bridge_weight_orientation():
    # W is [out, in]: output n reads row n of W
    h = np.array([[[1.0, 0.0, 0.0]]])
    wk = np.array([[0.5, 9.0, 9.0], [0.25, 9.0, 9.0]])
    kc, _, kx, _, _, _ = kv_bridge(h, wk, wk, 1.0, 1.0)
    assert kx.ravel().tolist() == [0.5, 0.25]
    assert TAB[kc.ravel()].tolist() == [0.5, 0.25]


def test_codes_follow_kernel_precision():
    # exact 1.0625 + 2^-30 lies above the midpoint between 1.0 and 1.125, but
    # its fp32 rounding is the midpoint itself, which rounds to even (1.0)
    x = np.array([1.0625 + 2.0 ** -30])
    assert encode_e4m3(x).tolist() == [57]
    assert quantize_kernel_precision(x, 1.0).tolist() == [56]
