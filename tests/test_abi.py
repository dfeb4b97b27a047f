"""The C-ABI library on the host: it loads, exports every declared symbol, and
rejects invalid arguments with the documented status before any GPU work.

No call here reaches a kernel launch: every case fails validation or is a
workspace-size query, so the tests run without a GPU.
"""
import ctypes
import os
import re

import pytest

from hybrid_sparse_attention_flash_amd import _lib
from hybrid_sparse_attention_flash_amd._lib import (HysAttnParams, HysDecodeParams, HysScoreParams, HysSparseParams,
                                                    HysTensor4)

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
INVALID, UNSUPPORTED, WORKSPACE = 1, 2, 3
FAKE = 0x7f0000000000          # 16-byte aligned, never dereferenced (validation fails first)


def lib():
    return _lib.load()


def t4(shape, dtype=1, strides=None, ptr=FAKE):
    t = HysTensor4()
    t.ptr = ptr
    t.dtype = dtype
    if strides is None:
        strides = [shape[1] * shape[2] * shape[3], shape[2] * shape[3], shape[3], 1]
    for i in range(4):
        t.shape[i] = shape[i]
        t.stride[i] = strides[i]
    return t


def test_exports_every_declared_symbol():
    hdr = open(os.path.join(ROOT, "include", "hys.h")).read()
    declared = set(re.findall(r"HYS_API[^;]*?\b(hys_\w+)\(", hdr))
    assert declared == set(_lib.EXPORTED)
    for name in declared:
        assert hasattr(lib(), name)
    assert lib().hys_abi_version() == 6
    assert lib().hys_status_string(3) == b"HYS_ERR_WORKSPACE"


def _full(p, q, k, v, o, sp=None, scores=None, ws=None, nb=None):
    nb = nb if nb is not None else ctypes.c_size_t(0)
    return lib().hys_full_attn_fwd(ctypes.byref(p), q, k, v, o, None, ctypes.byref(sp) if sp else None,
                                   scores, ws, ctypes.byref(nb), None)


def test_full_attn_validation():
    p = HysAttnParams(0.125, 1.0, 1.0)
    q, kv = t4([1, 128, 8, 128]), t4([1, 128, 2, 128])
    o = t4([1, 128, 8, 128], dtype=0)
    assert _full(p, HysTensor4(), kv, kv, o) == INVALID
    assert b"null" in lib().hys_last_error()
    assert _full(p, t4([1, 128, 8, 96]), t4([1, 128, 2, 96]), t4([1, 128, 2, 96]), t4([1, 128, 8, 96])) == UNSUPPORTED
    assert _full(p, q, t4([1, 128, 3, 128]), t4([1, 128, 3, 128]), o) == INVALID          # Hq % Hkv
    assert _full(p, q, t4([1, 128, 2, 128], strides=[0, 0, 128, 2]), kv, o) == INVALID   # d stride
    assert _full(p, q, kv, kv, t4([1, 127, 8, 128], dtype=0)) == INVALID                 # o shape
    assert _full(p, t4([1, 128, 8, 128], ptr=FAKE + 4), kv, kv, o) == INVALID            # alignment
    assert _full(p, q, t4([1, 128, 2, 128], dtype=0), t4([1, 128, 2, 128], dtype=0), o) == UNSUPPORTED  # bf16 q, f32 kv
    assert _full(HysAttnParams(float("nan"), 1, 1), q, kv, kv, o) == INVALID
    sp = HysScoreParams(1, 32)
    assert _full(p, q, kv, kv, o, sp, ctypes.c_void_p(FAKE)) == UNSUPPORTED               # block size 32
    sp = HysScoreParams(1, 64)
    assert _full(p, q, kv, kv, o, sp, None) == INVALID                                    # scores missing
    # workspace query: 2 KV groups x B x L x nblk floats
    nb = ctypes.c_size_t(0)
    assert _full(p, q, kv, kv, o, sp, ctypes.c_void_p(FAKE), None, nb) == 0
    assert nb.value == 2 * 1 * 128 * 2 * 4
    nb = ctypes.c_size_t(16)
    assert _full(p, q, kv, kv, o, sp, ctypes.c_void_p(FAKE), ctypes.c_void_p(FAKE), nb) == WORKSPACE


def test_topk_validation():
    L = lib()
    nb = ctypes.c_size_t(0)
    assert L.hys_select_topk(None, 4, 10, 10, -1, None, None, None, ctypes.byref(nb), None) == INVALID
    assert L.hys_select_topk(None, 4, 10, 5, 3, None, None, None, ctypes.byref(nb), None) == INVALID
    assert L.hys_select_topk(None, 4, 10, 10, 5000, None, None, None, ctypes.byref(nb), None) == UNSUPPORTED
    assert L.hys_select_topk(None, 4, 1 << 20, 1 << 20, 1024, None, None, None, ctypes.byref(nb), None) == 0
    # per row: 5120 histogram bins + 8 state words + 2 counts per chunk (128 chunks of 8192 columns)
    assert nb.value == 4 * (5120 + 8 + 2 * 128) * 4
    assert L.hys_select_topk(None, 2, 3000001, 3000001, 16, None, None, None, ctypes.byref(nb), None) == 0
    assert nb.value == 2 * (5120 + 8 + 2 * 367) * 4
    assert L.hys_select_topk(None, 1, (1 << 31) - 1, (1 << 31) - 1, 16, None, None, None, ctypes.byref(nb), None) == 0
    assert nb.value == (5120 + 8 + 2 * 1024) * 4        # at most 1024 chunks per row
    assert L.hys_select_topk(None, 4, 1 << 20, 1 << 20, 8192, None, None, None, ctypes.byref(nb), None) == UNSUPPORTED
    nb = ctypes.c_size_t(0)
    assert L.hys_select_topk(None, 4, 100, 100, 8, None, None, ctypes.c_void_p(FAKE), ctypes.byref(nb), None) == INVALID


def test_select_topk_blocks_validation():
    L = lib()
    nb = ctypes.c_size_t(0)

    def call(rows=4, cols=1000, stride=1000, block=64, kb=3, ws=None, idx=None):
        return L.hys_select_topk_blocks(None, rows, cols, stride, block, kb, idx, ws, ctypes.byref(nb), None)
    assert call(rows=-1) == INVALID
    assert call(cols=0) == INVALID
    assert call(stride=999) == INVALID
    assert call(block=32) == UNSUPPORTED
    assert call(kb=0) == UNSUPPORTED
    assert call(kb=33) == UNSUPPORTED
    # workspace: block maxima [rows, nblk] + block ids [rows, kb] + the top-k scratch, each 256-byte aligned
    assert call() == 0
    assert nb.value >= 256 + 256
    need = nb.value
    nb.value = need - 1
    assert call(ws=ctypes.c_void_p(FAKE)) == WORKSPACE
    nb.value = need
    assert call(ws=ctypes.c_void_p(FAKE)) == INVALID                  # null scores / idx


def test_group_stride_validation():
    p = HysAttnParams(0.125, 1.0, 1.0)
    q, kv, o = t4([1, 128, 8, 128]), t4([1, 128, 2, 128]), t4([1, 128, 8, 128], dtype=0)

    def sparse(sp):
        return lib().hys_sparse_attn_fwd(ctypes.byref(p), q, kv, kv, ctypes.byref(sp), ctypes.c_void_p(FAKE), o,
                                         None, None, None, None)

    def layer(sp):
        return lib().hys_sparse_layer_fwd(ctypes.byref(p), q, kv, kv, ctypes.byref(sp), ctypes.c_void_p(FAKE), kv, kv,
                                          128, ctypes.c_void_p(FAKE), None, o, None)
    assert sparse(HysSparseParams(64, 4, 1, 0, 512, 4, -1)) == INVALID
    assert sparse(HysSparseParams(1, 16, 64, 128, 32, 16, 64)) == UNSUPPORTED          # per-group sets need blocks
    assert layer(HysSparseParams(64, 4, 1, 0, 512, 4, -1)) == INVALID


def test_sparse_validation():
    p = HysAttnParams(0.125, 1.0, 1.0)
    q, kv, o = t4([1, 128, 8, 128]), t4([1, 128, 1, 128]), t4([1, 128, 8, 128], dtype=0)

    def call(sp, idx=FAKE):
        return lib().hys_sparse_attn_fwd(ctypes.byref(p), q, kv, kv, ctypes.byref(sp), ctypes.c_void_p(idx), o,
                                         None, None, None, None)
    assert call(HysSparseParams(32, 4, 1, 0, 512, 4)) == UNSUPPORTED
    assert call(HysSparseParams(64, 4, 64, 0, 512, 4)) == UNSUPPORTED
    assert call(HysSparseParams(64, 65, 1, 0, 512 * 65, 65)) == UNSUPPORTED
    assert call(HysSparseParams(64, 4, 1, 0, 512, 2)) == INVALID
    assert call(HysSparseParams(1, 4096, 64, 128, 8192, 4096)) == UNSUPPORTED
    assert call(HysSparseParams(1, 16, 64, 4000, 32, 16)) == UNSUPPORTED
    assert call(HysSparseParams(64, 4, 1, 0, 512, 4), idx=0) == INVALID


def test_sparse_layer_validation():
    p = HysAttnParams(0.125, 1.0, 1.0)
    q, kv, o = t4([1, 128, 8, 128]), t4([1, 128, 2, 128]), t4([1, 128, 8, 128], dtype=0)
    sp = HysSparseParams(64, 4, 1, 0, 512, 4)

    def call(q=q, k=kv, v=kv, kw=kv, vw=kv, sp=sp, idx=FAKE, window=128, gate=FAKE, o=o, p=p):
        return lib().hys_sparse_layer_fwd(ctypes.byref(p), q, k, v, ctypes.byref(sp), ctypes.c_void_p(idx), kw, vw,
                                          window, ctypes.c_void_p(gate), None, o, None)
    assert call(p=HysAttnParams(0.125, 2.0, 1.0)) == UNSUPPORTED                          # k_scale != 1
    assert call(k=t4([1, 128, 2, 128], dtype=2), v=t4([1, 128, 2, 128], dtype=2)) == UNSUPPORTED   # fp8 k/v
    assert call(kw=t4([1, 128, 2, 128], dtype=0), vw=t4([1, 128, 2, 128], dtype=0)) == UNSUPPORTED  # f32 window
    assert call(kw=t4([1, 128, 4, 64]), vw=t4([1, 128, 4, 64])) == INVALID               # head dims differ
    assert call(kw=t4([1, 128, 2, 128], strides=[2 * 128 * 128 + 128, 256, 128, 1])) == UNSUPPORTED  # strides
    assert call(sp=HysSparseParams(1, 16, 64, 128, 32, 16)) == UNSUPPORTED               # granularity 1
    assert call(sp=HysSparseParams(64, 65, 1, 0, 512 * 65, 65)) == UNSUPPORTED           # k > 64
    assert call(idx=0) == INVALID
    assert call(gate=0) == INVALID
    assert call(window=0) == INVALID
    assert call(o=t4([1, 128, 8, 64], dtype=0)) == INVALID                               # o shape


def test_decode_validation():
    p = HysDecodeParams(0.088, 0.01, 0.01, 1024, 128)
    qf = t4([4, 1, 64, 128])
    kc = t4([4, 1 << 20, 1, 128], dtype=2)
    o = t4([4, 1, 64, 128], dtype=0)
    lens = (ctypes.c_int64 * 4)(1 << 20, 1 << 20, 5, 1 << 20)
    nb = ctypes.c_size_t(0)

    def call(pp=p, q=qf, k=kc, ln=lens, n_sparse=0):
        return lib().hys_decode_step(ctypes.byref(pp), q, k, k, ln, o, ctypes.c_void_p(FAKE), ctypes.c_void_p(FAKE),
                                     n_sparse, None, None, None, ctypes.byref(nb), None)
    assert call() == 0 and nb.value > 0
    assert call(k=t4([4, 1 << 20, 2, 128], dtype=2)) == UNSUPPORTED          # not MQA
    assert call(q=t4([4, 1, 128, 128])) == INVALID or call(q=t4([4, 1, 128, 128])) == UNSUPPORTED
    bad = (ctypes.c_int64 * 4)(0, 1, 2, 3)
    assert call(ln=bad) == INVALID
    assert call(pp=HysDecodeParams(0.088, 0.01, 0.01, 4096, 128)) == UNSUPPORTED
    assert call(n_sparse=3) == INVALID                                        # null q_sparse


def test_kv_bridge_validation():
    from hybrid_sparse_attention_flash_amd._lib import HysBridgeParams
    p = HysBridgeParams(0.02, 0.02)
    h = t4([1, 300, 1, 4096])
    kc = t4([1, 300, 1, 128], dtype=2)

    def call(pp=p, h=h, k=kc, v=kc, wk=FAKE, wv=FAKE, amax=None):
        return lib().hys_kv_bridge_fwd(ctypes.byref(pp) if pp is not None else None, h, ctypes.c_void_p(wk),
                                       ctypes.c_void_p(wv), k, v, amax, None)
    assert call(pp=None) == INVALID
    assert call(pp=HysBridgeParams(0.0, 0.02)) == INVALID                     # scale 0
    assert call(pp=HysBridgeParams(float("nan"), 0.02)) == INVALID
    assert call(pp=HysBridgeParams(1e-45, 0.02)) == INVALID                   # reciprocal overflows
    assert call(h=t4([1, 300, 1, 4096], dtype=0)) == UNSUPPORTED               # fp32 hidden states
    assert call(h=t4([1, 300, 2, 4096])) == INVALID                           # H != 1
    assert call(h=t4([1, 300, 1, 4000])) == UNSUPPORTED                        # d_model % 64
    assert call(h=t4([1, 300, 1, 4096], strides=[300 * 4100, 4100, 4096, 1])) == INVALID   # token stride % 8
    assert call(k=t4([1, 300, 1, 128], dtype=1), v=t4([1, 300, 1, 128], dtype=1)) == UNSUPPORTED  # bf16 cache
    assert call(k=t4([1, 301, 1, 128], dtype=2), v=t4([1, 301, 1, 128], dtype=2)) == INVALID     # L differs
    assert call(v=t4([1, 300, 2, 128], dtype=2)) == INVALID                   # K/V shapes differ
    assert call(v=t4([1, 300, 1, 128], dtype=2, strides=[300 * 256, 256, 128, 1])) == UNSUPPORTED  # strides differ
    assert call(k=t4([1, 300, 1, 64], dtype=2), v=t4([1, 300, 1, 64], dtype=2)) == UNSUPPORTED   # Hkv*D = 64
    assert call(wk=0) == INVALID
    assert call(wv=FAKE + 8) == INVALID                                       # misaligned weights
    assert call(amax=ctypes.c_void_p(FAKE + 2)) == INVALID                    # misaligned amax
    assert b"amax" in lib().hys_last_error()


def test_kv_bridge_empty_accepts_null_tensors():
    """L = 0 with null tensor pointers and no amax passes validation and launches nothing."""
    from hybrid_sparse_attention_flash_amd._lib import HysBridgeParams
    p = HysBridgeParams(0.02, 0.02)
    h = t4([2, 0, 1, 128], ptr=0)
    kc = t4([2, 0, 1, 128], dtype=2, ptr=0)
    assert lib().hys_kv_bridge_fwd(ctypes.byref(p), h, ctypes.c_void_p(FAKE), ctypes.c_void_p(FAKE), kc, kc,
                                   None, None) == 0
    h1 = t4([2, 1, 1, 128], ptr=0)
    assert lib().hys_kv_bridge_fwd(ctypes.byref(p), h1, ctypes.c_void_p(FAKE), ctypes.c_void_p(FAKE), kc, kc,
                                   None, None) == INVALID


def test_hysparse_decode_validation():
    from hybrid_sparse_attention_flash_amd._lib import HysHsDecodeParams
    B, N, Hq, Hkv, D, W, nl = 2, 4096, 32, 4, 128, 128, 2
    p = HysHsDecodeParams(0.088, 16, 64)
    q = t4([B, 1, Hq, D])
    kc = t4([B, N, Hkv, D])
    o = t4([B, 1, Hq, D], dtype=0)
    lens = (ctypes.c_int64 * B)(N, 100)
    qs = (HysTensor4 * nl)(*[t4([B, 1, Hq, D]) for _ in range(nl)])
    new = (HysTensor4 * nl)(*[t4([B, 1, Hkv, D]) for _ in range(nl)])
    ring = (HysTensor4 * nl)(*[t4([B, W, Hkv, D]) for _ in range(nl)])
    gw = (ctypes.c_void_p * nl)(FAKE, FAKE)
    nb = ctypes.c_size_t(0)

    def call(pp=p, q=q, k=kc, ln=lens, n_sparse=nl, ring=ring, new=new, gw=gw, scores=FAKE):
        return lib().hys_hysparse_decode_step(ctypes.byref(pp), q, k, k, ln, o, ctypes.c_void_p(scores),
                                              ctypes.c_void_p(FAKE), n_sparse, qs, new, new, ring, ring, gw, qs,
                                              None, ctypes.byref(nb), None)
    assert call() == 0 and nb.value > 0                                         # size query
    assert call(k=t4([B, N, Hkv, D], dtype=2)) == UNSUPPORTED                   # fp8 cache
    assert call(q=t4([B, 1, 64, D]), k=t4([B, N, 2, D])) == UNSUPPORTED          # G = 32 > 16
    assert call(q=t4([B, 1, 12, D]), k=t4([B, N, 4, D])) == UNSUPPORTED          # G = 3
    assert call(pp=HysHsDecodeParams(0.088, 65, 64)) == UNSUPPORTED              # topk > 64
    assert call(pp=HysHsDecodeParams(0.088, 16, 32)) == UNSUPPORTED              # block != 64
    assert call(ln=(ctypes.c_int64 * B)(0, 5)) == INVALID                       # empty sequence
    assert call(ln=(ctypes.c_int64 * B)(N + 1, 5)) == INVALID                   # beyond the cache
    bad_ring = (HysTensor4 * nl)(*[t4([B, W, Hkv, 64]) for _ in range(nl)])
    assert call(ring=bad_ring) == INVALID                                       # ring head dim
    bad_new = (HysTensor4 * nl)(*[t4([B, 2, Hkv, D]) for _ in range(nl)])
    assert call(new=bad_new) == INVALID                                         # two new tokens
    assert call(gw=(ctypes.c_void_p * nl)(FAKE, 0)) == INVALID                  # null gate
    assert call(scores=0) == INVALID
    assert call(n_sparse=17) == UNSUPPORTED
    assert call(n_sparse=0) == 0                                                # full layer only


def test_backward_validation():
    L_ = lib()
    p = HysAttnParams(0.125, 1.0, 1.0)
    q, kv = t4([1, 128, 8, 128]), t4([1, 128, 2, 128])
    o, dq = t4([1, 128, 8, 128], dtype=0), t4([1, 128, 8, 128], dtype=0)
    dkv = t4([1, 128, 2, 128], dtype=0)
    nb = ctypes.c_size_t(0)

    def full(q=q, k=kv, v=kv, d_o=q, dq=dq, dk=dkv, dv=dkv, lse=FAKE, acc=0, p=p, ws=None):
        return L_.hys_full_attn_bwd(ctypes.byref(p), q, k, v, o, ctypes.c_void_p(lse) if lse else None, d_o, dq, dk,
                                    dv, acc, ws, ctypes.byref(nb), None)
    assert full() == 0 and nb.value >= 4 * 8 * 128                          # size query: rowsum(dO * O)
    assert full(p=HysAttnParams(0.125, 2.0, 1.0)) == UNSUPPORTED             # k_scale != 1
    assert full(q=t4([1, 128, 8, 128], dtype=0), d_o=t4([1, 128, 8, 128], dtype=0)) == UNSUPPORTED  # fp32 q
    assert full(d_o=t4([1, 128, 8, 128], dtype=0)) == UNSUPPORTED           # d_o must be bf16
    assert full(dq=t4([1, 128, 8, 128])) == UNSUPPORTED                     # bf16 gradient
    assert full(dk=t4([1, 127, 2, 128], dtype=0)) == INVALID                # dk shape
    assert full(dv=t4([1, 128, 2, 128], dtype=0, strides=[128 * 512, 512, 128, 1])) == UNSUPPORTED   # dk, dv strides
    assert full(lse=0) == INVALID
    assert full(acc=2) == INVALID
    need = nb.value
    nb.value = need - 1
    assert full(ws=ctypes.c_void_p(FAKE)) == WORKSPACE

    sp = HysSparseParams(64, 4, 1, 0, 512, 4, 0)

    def layer(sp=sp, window=128, gate=FAKE, dgate=FAKE, kw=kv, dkw=dkv, ws=None):
        nb.value = 0
        return L_.hys_sparse_layer_bwd(ctypes.byref(p), q, kv, kv, ctypes.byref(sp), ctypes.c_void_p(FAKE), kw, kw,
                                       window, ctypes.c_void_p(gate) if gate else None, None, o,
                                       ctypes.c_void_p(FAKE), o, ctypes.c_void_p(FAKE), q, dq, dkv, dkv, 1, dkw, dkw,
                                       ctypes.c_void_p(dgate) if dgate else None, None, ws, ctypes.byref(nb), None)
    assert layer() == 0 and nb.value > 2 * 2 * 128 * 8 * 128                  # two bf16 branch gradients
    assert layer(sp=HysSparseParams(1, 16, 64, 128, 32, 16, 0)) == UNSUPPORTED   # token granularity
    assert layer(sp=HysSparseParams(64, 65, 1, 0, 512 * 65, 65, 0)) == UNSUPPORTED
    assert layer(sp=HysSparseParams(64, 4, 1, 0, 512, 4, -1)) == INVALID
    assert layer(window=0) == INVALID
    assert layer(gate=0) == INVALID
    assert layer(dgate=0) == INVALID
    assert layer(kw=t4([1, 128, 2, 64]), dkw=t4([1, 128, 2, 64], dtype=0)) == INVALID   # head dims differ

    def window_fwd(window=128, o=o):
        return L_.hys_window_attn_fwd(ctypes.byref(p), q, kv, kv, window, o, None, None)
    assert window_fwd(window=0) == INVALID
    assert window_fwd(o=t4([1, 128, 8, 64], dtype=0)) == INVALID


def test_decode_noalloc_validation_and_scratch_limit():
    """The entry point without workspace validates like hys_decode_step and
    refuses a step whose workspace exceeds its fixed scratch, both before any
    HIP call."""
    L = lib()
    p = HysDecodeParams(0.088, 0.01, 0.01, 1024, 128)
    o = t4([4, 1, 64, 128], dtype=0)

    def call(B, N, lens, n_sparse=0, pp=p):
        qf = t4([B, 1, 64, 128])
        kc = t4([B, N, 1, 128], dtype=2)
        ob = t4([B, 1, 64, 128], dtype=0)
        arr = (HysTensor4 * max(n_sparse, 1))(*[t4([B, 1, 64, 128]) for _ in range(n_sparse)])
        arr_o = (HysTensor4 * max(n_sparse, 1))(*[t4([B, 1, 64, 128], dtype=0) for _ in range(n_sparse)])
        ln = (ctypes.c_int64 * B)(*lens)
        return L.hys_decode_step_noalloc(ctypes.byref(pp), qf, kc, kc, ln, ob, ctypes.c_void_p(FAKE),
                                         ctypes.c_void_p(FAKE), n_sparse, arr if n_sparse else None,
                                         arr_o if n_sparse else None, None)
    assert call(4, 1 << 20, [0, 1, 2, 3]) == INVALID                           # cache_len 0
    assert call(4, 1 << 20, [1 << 20] * 4, pp=HysDecodeParams(0.088, 0.01, 0.01, 4096, 128)) == UNSUPPORTED
    # 64 sequences x 16 sparse layers: the split partials alone exceed 64 MiB
    big = 16
    nb = ctypes.c_size_t(0)
    qf, kc = t4([64, 1, 64, 128]), t4([64, 4096, 1, 128], dtype=2)
    arr = (HysTensor4 * big)(*[t4([64, 1, 64, 128]) for _ in range(big)])
    arr_o = (HysTensor4 * big)(*[t4([64, 1, 64, 128], dtype=0) for _ in range(big)])
    ln = (ctypes.c_int64 * 64)(*([4096] * 64))
    assert L.hys_decode_step(ctypes.byref(p), qf, kc, kc, ln, t4([64, 1, 64, 128], dtype=0), ctypes.c_void_p(FAKE),
                             ctypes.c_void_p(FAKE), big, arr, arr_o, None, ctypes.byref(nb), None) == 0
    assert nb.value > 64 << 20
    assert call(64, 4096, [4096] * 64, n_sparse=big) == WORKSPACE
    assert b"scratch" in L.hys_last_error()


def test_attn_params_causal_and_q_offset():
    """hys_attn_params carries causal (must be 1) and q_offset (row 0's absolute
    position, q_offset + Lq <= Lk); the backward calls take q_offset 0 only."""
    import ctypes as C
    assert C.sizeof(HysAttnParams) == 24 and HysAttnParams.q_offset.offset == 16
    q, kv = t4([1, 64, 8, 128]), t4([1, 256, 2, 128])
    o = t4([1, 64, 8, 128], dtype=0)
    assert _full(HysAttnParams(0.125, 1.0, 1.0, 1, 192), q, kv, kv, o) == 0          # chunk of a 256-token cache
    assert _full(HysAttnParams(0.125, 1.0, 1.0, 1, 193), q, kv, kv, o) == INVALID    # 193 + 64 > 256
    assert _full(HysAttnParams(0.125, 1.0, 1.0, 0, 0), q, kv, kv, o) == UNSUPPORTED  # non-causal
    assert b"causal" in lib().hys_last_error()
    assert _full(HysAttnParams(0.125, 1.0, 1.0, 1, -1), q, kv, kv, o) == INVALID
    # score sizes follow the key length: BLOCK with 2 KV groups needs Hkv*B*Lq*ceil(Lk/64) floats
    sp = HysScoreParams(1, 64)
    nb = C.c_size_t(0)
    assert _full(HysAttnParams(0.125, 1.0, 1.0, 1, 100), q, kv, kv, o, sp, C.c_void_p(FAKE), None, nb) == 0
    assert nb.value == 2 * 1 * 64 * 4 * 4
    # the backward pass refuses an offset
    L = lib()
    qb, kb = t4([1, 64, 8, 128]), t4([1, 64, 2, 128])
    of = t4([1, 64, 8, 128], dtype=0)
    kf = t4([1, 64, 2, 128], dtype=0)
    args = [C.byref(HysAttnParams(0.125, 1.0, 1.0, 1, 3)), qb, kb, kb, qb, C.c_void_p(FAKE), qb, of, kf, kf, 0,
            None, C.byref(nb), None]
    assert L.hys_full_attn_bwd(*args) == UNSUPPORTED
