"""Valid calls of every entry point, on a host without a GPU.

Each call below passes validation, so the library derives its launch
configuration (work decomposition, grid, score and workspace layout) and only
the launch itself fails, for want of a device: the status is HYS_ERR_HIP.  In
the host-checked build (tests/test_checked_build.py: -DHYS_DEBUG, host ASan and
UBSan) the launch-arithmetic checks run on every one of these configurations
before that, so a broken invariant shows up as HYS_ERR_INTERNAL and an
out-of-bounds or undefined host operation as a sanitizer abort.

The tensors are fake, never dereferenced addresses: this module must never run
where a GPU is visible (a launch would then read them), and it skips itself
there.
"""
import ctypes
import os
import sys

import pytest

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
from test_abi import FAKE, lib, t4  # noqa: E402

from hybrid_sparse_attention_flash_amd._lib import (HysAttnParams, HysBridgeParams, HysDecodeParams,  # noqa: E402
                                                    HysHsDecodeParams, HysScoreParams, HysSparseParams, HysTensor4)

HIP_ERR = 4
F32, BF16, FP8 = 0, 1, 2


def _device_visible():
    for name in ("libamdhip64.so", "libamdhip64.so.7", "libamdhip64.so.6"):
        try:
            hip = ctypes.CDLL(name)
        except OSError:
            continue
        n = ctypes.c_int(0)
        return hip.hipGetDeviceCount(ctypes.byref(n)) == 0 and n.value > 0
    return False


pytestmark = pytest.mark.skipif(_device_visible(), reason="fake-pointer launches are for GPU-less hosts only")


def reaches_launch(status):
    msg = lib().hys_last_error().decode()
    assert status == HIP_ERR, f"status {status}: {msg}"
    assert "launch check failed" not in msg


def ws_of(fn):
    """Query the workspace size, then call with a fake workspace of that size."""
    nb = ctypes.c_size_t(0)
    st = fn(None, nb)
    assert st == 0, lib().hys_last_error().decode()
    return fn(ctypes.c_void_p(FAKE), nb)


FULL_CASES = [
    # B, Lq, Lk, Hq, Hkv, D, q dtype, kv dtype, score mode, q_offset
    (1, 1024, 1024, 8, 1, 64, F32, F32, 1, 0),             # tiny fp32 block
    (1, 16384, 16384, 32, 8, 128, BF16, BF16, 1, 0),       # dense 7B-class, 16k
    (1, 32768, 32768, 32, 4, 128, BF16, BF16, 1, 0),       # MoE 80B-class, 32k
    (1, 32768, 32768, 32, 4, 128, BF16, BF16, 3, 0),       # per-KV-group block scores
    (1, 65536, 65536, 64, 1, 128, BF16, FP8, 2, 0),        # HySparse2 64k tile-token scores
    (2, 300, 301, 16, 16, 64, BF16, BF16, 0, 1),           # G = 1, ragged, chunk at an offset
    (3, 77, 4173, 24, 8, 128, BF16, FP8, 1, 4096),         # G = 3, chunked prefill
    (1, 513, 513, 128, 1, 128, BF16, BF16, 1, 0),          # G = 128
    (1, 200, 1000, 8, 1, 128, BF16, BF16, 2, 800),         # tile-token scores of a chunk
    (1, 1, 1, 4, 2, 64, F32, F32, 1, 0),                   # one query
]


@pytest.mark.parametrize("case", FULL_CASES)
def test_full_attention_configs(case):
    B, Lq, Lk, Hq, Hkv, D, qd, kd, mode, q_off = case
    p = HysAttnParams(D ** -0.5, q_offset=q_off)
    q, kv, o = t4([B, Lq, Hq, D], qd), t4([B, Lk, Hkv, D], kd), t4([B, Lq, Hq, D], F32)
    sp = HysScoreParams(mode, 64)
    scores = ctypes.c_void_p(FAKE) if mode else None
    reaches_launch(ws_of(lambda ws, nb: lib().hys_full_attn_fwd(ctypes.byref(p), q, kv, kv, o, None, ctypes.byref(sp),
                                                                 scores, ws, ctypes.byref(nb), None)))


SPARSE_CASES = [
    # B, Lq, Lk, Hq, Hkv, D, q dtype, kv dtype, granularity, k, q_tile, forced window, q_offset, group sets
    (1, 32768, 32768, 32, 4, 128, BF16, BF16, 64, 16, 1, 0, 0, False),
    (1, 32768, 32768, 32, 4, 128, BF16, BF16, 64, 16, 1, 0, 0, True),
    (1, 16384, 16384, 32, 8, 128, BF16, FP8, 64, 64, 1, 0, 0, False),
    (2, 333, 1000, 6, 2, 64, F32, F32, 64, 5, 1, 0, 667, False),
    (1, 65536, 65536, 64, 1, 128, BF16, FP8, 1, 1024, 64, 128, 0, False),
    (1, 700, 828, 8, 1, 128, BF16, BF16, 1, 2048, 64, 1984, 128, False),
    (1, 64, 64, 2, 2, 64, BF16, BF16, 1, 1, 64, 0, 0, False),
]


@pytest.mark.parametrize("case", SPARSE_CASES)
def test_sparse_attention_configs(case):
    B, Lq, Lk, Hq, Hkv, D, qd, kd, gran, k, qt, fw, q_off, groups = case
    p = HysAttnParams(D ** -0.5, q_offset=q_off)
    q, kv, o = t4([B, Lq, Hq, D], qd), t4([B, Lk, Hkv, D], kd), t4([B, Lq, Hq, D], F32)
    rows = Lq if gran == 64 else (Lq + 63) // 64
    sp = HysSparseParams(gran, k, qt, fw, rows * k, k, (B * rows * k) if groups else 0)
    reaches_launch(lib().hys_sparse_attn_fwd(ctypes.byref(p), q, kv, kv, ctypes.byref(sp), ctypes.c_void_p(FAKE), o,
                                             ctypes.c_void_p(FAKE), None, None, None))


LAYER_CASES = [
    # B, Lq, Lk, Hq, Hkv, D, dtype, k, window, q_offset, out dtype
    (1, 32768, 32768, 32, 4, 128, BF16, 16, 128, 0, BF16),   # the one-pass layer of the MoE 32k block
    (1, 16384, 16384, 32, 8, 128, BF16, 16, 128, 0, F32),
    (1, 1024, 1024, 8, 1, 64, F32, 4, 128, 0, F32),           # engine path (fp32)
    (2, 257, 400, 16, 4, 128, BF16, 2, 40, 143, BF16),
    (1, 150, 150, 32, 2, 128, BF16, 5, 128, 0, BF16),
    (1, 100, 100, 3, 1, 64, BF16, 64, 1, 0, F32),             # G = 3, k = 64, window 1
]


@pytest.mark.parametrize("case", LAYER_CASES)
def test_sparse_layer_configs(case):
    B, Lq, Lk, Hq, Hkv, D, dt, k, W, q_off, od = case
    p = HysAttnParams(D ** -0.5, q_offset=q_off)
    q, kv, o = t4([B, Lq, Hq, D], dt), t4([B, Lk, Hkv, D], dt), t4([B, Lq, Hq, D], od)
    sp = HysSparseParams(64, k, 1, 0, Lq * k, k, 0)
    reaches_launch(lib().hys_sparse_layer_fwd(ctypes.byref(p), q, kv, kv, ctypes.byref(sp), ctypes.c_void_p(FAKE), kv,
                                              kv, W, ctypes.c_void_p(FAKE), None, o, None))


@pytest.mark.parametrize("case", [(1, 32768, 32, 4, 128, 128, BF16), (2, 300, 8, 8, 64, 1, FP8),
                                  (1, 65536, 64, 1, 128, 128, FP8)])
def test_swa_gate_and_window_configs(case):
    B, L, Hq, Hkv, D, W, kd = case
    p = HysAttnParams(D ** -0.5)
    q, kv, o = t4([B, L, Hq, D], BF16), t4([B, L, Hkv, D], kd), t4([B, L, Hq, D], F32)
    reaches_launch(lib().hys_swa_gate_fwd(ctypes.byref(p), q, kv, kv, W, o, ctypes.c_void_p(FAKE),
                                          ctypes.c_void_p(FAKE), None, o, None))
    reaches_launch(lib().hys_window_attn_fwd(ctypes.byref(p), q, kv, kv, W, o, ctypes.c_void_p(FAKE), None))


@pytest.mark.parametrize("rows, cols, k", [(32768, 512, 16), (4, 1 << 20, 1024), (4, (1 << 20) + 4096, 1024),
                                           (1, 3000001, 2048), (65536, 1024, 1), (3, 40000, 7)])
def test_topk_configs(rows, cols, k):
    reaches_launch(ws_of(lambda ws, nb: lib().hys_select_topk(ctypes.c_void_p(FAKE), rows, cols, cols, k,
                                                               ctypes.c_void_p(FAKE), None, ws, ctypes.byref(nb),
                                                               None)))
    if k <= 32:
        reaches_launch(ws_of(lambda ws, nb: lib().hys_select_topk_blocks(ctypes.c_void_p(FAKE), rows, cols, cols, 64,
                                                                          k, ctypes.c_void_p(FAKE), ws,
                                                                          ctypes.byref(nb), None)))


@pytest.mark.parametrize("case", [(4, 1 << 20, (1 << 20, 1 << 20, 1 << 20, 1 << 20), 64, 11, FP8),
                                  (4, (1 << 20) + 4096, ((1 << 20) + 4096, 1 << 20, 524289, 3), 64, 3, BF16),
                                  (1, 5000, (5000,), 8, 0, BF16), (16, 70000, tuple(1 + 4371 * i for i in range(16)), 16, 2, FP8)])
def test_decode_configs(case):
    B, N, lens, Hq, nsp, kd = case
    lens = (ctypes.c_int64 * B)(*lens)
    p = HysDecodeParams(128 ** -0.5, 1.0, 1.0, 1024 if N >= 1024 else 256, 128)
    qf, cache, of = t4([B, 1, Hq, 128], BF16), t4([B, N, 1, 128], kd), t4([B, 1, Hq, 128], F32)
    qs = (HysTensor4 * max(nsp, 1))(*([t4([B, 1, Hq, 128], BF16)] * max(nsp, 1)))
    os_ = (HysTensor4 * max(nsp, 1))(*([t4([B, 1, Hq, 128], F32)] * max(nsp, 1)))

    def call(ws, nb):
        return lib().hys_decode_step(ctypes.byref(p), qf, cache, cache, lens, of, ctypes.c_void_p(FAKE),
                                     ctypes.c_void_p(FAKE), nsp, qs, os_, ws, ctypes.byref(nb), None)
    reaches_launch(ws_of(call))


def test_kv_bridge_config():
    p = HysBridgeParams(1.0, 1.0)
    h = t4([1, 65536, 1, 4096], BF16, strides=[65536 * 4096, 4096, 4096, 1])
    kc = t4([1, 65536, 1, 128], FP8)
    reaches_launch(lib().hys_kv_bridge_fwd(ctypes.byref(p), h, ctypes.c_void_p(FAKE), ctypes.c_void_p(FAKE), kc, kc,
                                           ctypes.c_void_p(FAKE), None))


def test_hysparse_decode_config():
    B, N, Hq, Hkv, D, W, nsp = 4, 131072, 32, 4, 128, 128, 11
    p = HysHsDecodeParams(D ** -0.5, 16, 64)
    lens = (ctypes.c_int64 * B)(N, N - 1, 70000, 64)
    qf, of = t4([B, 1, Hq, D], BF16), t4([B, 1, Hq, D], F32)
    cache = t4([B, N, Hkv, D], BF16)
    qs = (HysTensor4 * nsp)(*[t4([B, 1, Hq, D], BF16) for _ in range(nsp)])
    new = (HysTensor4 * nsp)(*[t4([B, 1, Hkv, D], BF16) for _ in range(nsp)])
    ring = (HysTensor4 * nsp)(*[t4([B, W, Hkv, D], BF16) for _ in range(nsp)])
    os_ = (HysTensor4 * nsp)(*[t4([B, 1, Hq, D], F32) for _ in range(nsp)])
    gw = (ctypes.c_void_p * nsp)(*([FAKE] * nsp))

    def call(ws, nb):
        return lib().hys_hysparse_decode_step(ctypes.byref(p), qf, cache, cache, lens, of, ctypes.c_void_p(FAKE),
                                              ctypes.c_void_p(FAKE), nsp, qs, new, new, ring, ring, gw, os_, ws,
                                              ctypes.byref(nb), None)
    reaches_launch(ws_of(call))
