"""Python binding of the C-ABI calls (argument marshalling only).

PyTorch supplies device memory and the current stream; every computation runs
in libhys.so.  Workspace, when a call needs one, is queried from the library
and allocated with torch on the same device.
"""
import ctypes
import math
from typing import List, Optional, Sequence

import torch

from . import _lib
from ._lib import (HYS_BF16, HYS_F32, HYS_FP8_E4M3, HYS_SCORE_BLOCK, HYS_SCORE_BLOCK_GROUP, HYS_SCORE_NONE,
                   HYS_SCORE_TILE_TOKEN,
                   HysAttnParams, HysBridgeParams, HysDecodeParams, HysHsDecodeParams, HysScoreParams, HysSparseParams, HysTensor4, check)

_DT = {torch.float32: HYS_F32, torch.bfloat16: HYS_BF16, torch.uint8: HYS_FP8_E4M3,
       torch.float8_e4m3fn: HYS_FP8_E4M3}
_SCORE = {"none": HYS_SCORE_NONE, "block": HYS_SCORE_BLOCK, "tile_token": HYS_SCORE_TILE_TOKEN,
          "block_group": HYS_SCORE_BLOCK_GROUP}


def tensor4(t: torch.Tensor) -> HysTensor4:
    """Describe a [B, T, H, D] torch tensor (fp8 given as uint8 or float8_e4m3fn)."""
    if t.dim() != 4:
        raise ValueError(f"expected a 4-D [B, T, H, D] tensor, got shape {tuple(t.shape)}")
    if t.dtype not in _DT:
        raise TypeError(f"unsupported dtype {t.dtype}")
    d = HysTensor4()
    d.ptr = t.data_ptr()
    d.dtype = _DT[t.dtype]
    for i in range(4):
        d.shape[i] = t.shape[i]
        d.stride[i] = t.stride(i)
    return d


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _workspace(nbytes: int, device) -> torch.Tensor:
    # ws == NULL means "size query", so a run always passes a real buffer
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)


def hys_full_attn_fwd(q, k, v, o, lse=None, score_mode: str = "none", scores=None, softmax_scale: float = None,
                      k_scale: float = 1.0, v_scale: float = 1.0, score_size: int = 64, q_offset: int = 0):
    """q_offset: absolute position of q's row 0 (chunked prefill: k, v may be
    longer than q, with q_offset + Lq <= Lk)."""
    lib = _lib.load()
    p = HysAttnParams(softmax_scale or 1.0 / math.sqrt(q.shape[-1]), k_scale, v_scale, q_offset=q_offset)
    sp = HysScoreParams(_SCORE[score_mode], score_size)
    args = [ctypes.byref(p), tensor4(q), tensor4(k), tensor4(v), tensor4(o), _ptr(lse), ctypes.byref(sp),
            _ptr(scores)]
    nb = ctypes.c_size_t(0)
    check(lib.hys_full_attn_fwd(*args, None, ctypes.byref(nb), None))
    ws = _workspace(nb.value, q.device)
    nb = ctypes.c_size_t(ws.numel())
    check(lib.hys_full_attn_fwd(*args, _ptr(ws), ctypes.byref(nb), _stream(q.device)))
    return ws


def hys_select_topk(scores: torch.Tensor, k: int, idx: torch.Tensor, count: Optional[torch.Tensor] = None):
    """scores: 2-D fp32 [rows, cols] (row stride from the tensor); idx [rows, k] int32 contiguous."""
    lib = _lib.load()
    rows, cols = scores.shape
    args = [_ptr(scores), rows, cols, scores.stride(0) if rows > 0 else cols, k, _ptr(idx), _ptr(count)]
    nb = ctypes.c_size_t(0)
    check(lib.hys_select_topk(*args, None, ctypes.byref(nb), None))
    ws = _workspace(nb.value, scores.device)
    nb = ctypes.c_size_t(ws.numel())
    check(lib.hys_select_topk(*args, _ptr(ws), ctypes.byref(nb), _stream(scores.device)))
    return ws


def hys_select_topk_blocks(scores: torch.Tensor, k_blocks: int, idx: torch.Tensor, block: int = 64):
    """scores: 2-D fp32 [rows, cols]; idx [rows, 64 * k_blocks] int32 contiguous: the top k_blocks blocks'
    token positions (ascending, -1 padded)."""
    lib = _lib.load()
    rows, cols = scores.shape
    args = [_ptr(scores), rows, cols, scores.stride(0) if rows > 0 else cols, block, k_blocks, _ptr(idx)]
    nb = ctypes.c_size_t(0)
    check(lib.hys_select_topk_blocks(*args, None, ctypes.byref(nb), None))
    ws = _workspace(nb.value, scores.device)
    nb = ctypes.c_size_t(ws.numel())
    check(lib.hys_select_topk_blocks(*args, _ptr(ws), ctypes.byref(nb), _stream(scores.device)))
    return ws


def hys_sparse_attn_fwd(q, k, v, idx, o, lse=None, granularity: int = 64, topk: int = None, q_tile: int = 1,
                        forced_window: int = 0, softmax_scale: float = None, k_scale: float = 1.0,
                        v_scale: float = 1.0, q_offset: int = 0):
    """idx: [B, R, topk] int32 (R = L for q_tile 1, ceil(L/64) for q_tile 64), or
    [Hkv, B, L, topk] for per-KV-group index sets (granularity 64)."""
    lib = _lib.load()
    p = HysAttnParams(softmax_scale or 1.0 / math.sqrt(q.shape[-1]), k_scale, v_scale, q_offset=q_offset)
    kk = idx.shape[-1] if topk is None else topk
    gs, ib = (idx.stride(0), idx[0]) if idx.dim() == 4 else (0, idx)
    sp = HysSparseParams(granularity, kk, q_tile, forced_window, ib.stride(0), ib.stride(1), gs)
    check(lib.hys_sparse_attn_fwd(ctypes.byref(p), tensor4(q), tensor4(k), tensor4(v), ctypes.byref(sp), _ptr(idx),
                                  tensor4(o), _ptr(lse), None, None, _stream(q.device)))


def hys_swa_gate_fwd(q, k_win, v_win, window: int, o_sparse, lse_sparse, gate_w, o, gate_b=None,
                     softmax_scale: float = None, k_scale: float = 1.0, v_scale: float = 1.0, q_offset: int = 0):
    lib = _lib.load()
    p = HysAttnParams(softmax_scale or 1.0 / math.sqrt(q.shape[-1]), k_scale, v_scale, q_offset=q_offset)
    check(lib.hys_swa_gate_fwd(ctypes.byref(p), tensor4(q), tensor4(k_win), tensor4(v_win), window,
                               tensor4(o_sparse), _ptr(lse_sparse), _ptr(gate_w), _ptr(gate_b), tensor4(o),
                               _stream(q.device)))


def hys_sparse_layer_fwd(q, k, v, idx, k_win, v_win, window: int, gate_w, o, gate_b=None, topk: int = None,
                         softmax_scale: float = None, q_offset: int = 0):
    """One HySparse sparse layer (selected blocks of k/v, own window k_win/v_win, sigmoid gate) in one call.
    idx: [B, L, topk] int32 block ids, or [Hkv, B, L, topk] for per-KV-group index sets."""
    lib = _lib.load()
    p = HysAttnParams(softmax_scale or 1.0 / math.sqrt(q.shape[-1]), 1.0, 1.0, q_offset=q_offset)
    kk = idx.shape[-1] if topk is None else topk
    gs, ib = (idx.stride(0), idx[0]) if idx.dim() == 4 else (0, idx)
    sp = HysSparseParams(64, kk, 1, 0, ib.stride(0), ib.stride(1), gs)
    check(lib.hys_sparse_layer_fwd(ctypes.byref(p), tensor4(q), tensor4(k), tensor4(v), ctypes.byref(sp), _ptr(idx),
                                   tensor4(k_win), tensor4(v_win), window, _ptr(gate_w), _ptr(gate_b), tensor4(o),
                                   _stream(q.device)))


def hys_decode_step_args(q_full, k_cache, v_cache, cache_len: Sequence[int], o_full, token_scores, idx,
                         q_sparse: Sequence[torch.Tensor], o_sparse: Sequence[torch.Tensor], topk: int, window: int,
                         softmax_scale: float = None, k_scale: float = 1.0, v_scale: float = 1.0,
                         workspace: Optional[torch.Tensor] = None):
    """The marshalled arguments of one hys_decode_step call and the workspace
    they use (allocated here when `workspace` is missing or too small): the
    call is lib.hys_decode_step(*args).  The ctypes objects the tuple refers
    to live as long as the tuple."""
    lib = _lib.load()
    p = HysDecodeParams(softmax_scale or 1.0 / math.sqrt(q_full.shape[-1]), k_scale, v_scale, topk, window)
    lens = (ctypes.c_int64 * len(cache_len))(*[int(x) for x in cache_len])
    n = len(q_sparse)
    qs = (HysTensor4 * max(n, 1))(*[tensor4(t) for t in q_sparse])
    os_ = (HysTensor4 * max(n, 1))(*[tensor4(t) for t in o_sparse])
    args = [ctypes.byref(p), tensor4(q_full), tensor4(k_cache), tensor4(v_cache), lens, tensor4(o_full),
            _ptr(token_scores), _ptr(idx), n, qs, os_]
    nb = ctypes.c_size_t(0)
    check(lib.hys_decode_step(*args, None, ctypes.byref(nb), None))
    if workspace is None or workspace.numel() < nb.value:
        workspace = _workspace(nb.value, q_full.device)
    nb2 = ctypes.c_size_t(workspace.numel())
    return tuple(args) + (_ptr(workspace), ctypes.byref(nb2), _stream(q_full.device)), workspace, (p, lens, qs, os_, nb2)


def hys_decode_step(q_full, k_cache, v_cache, cache_len: Sequence[int], o_full, token_scores, idx,
                    q_sparse: Sequence[torch.Tensor], o_sparse: Sequence[torch.Tensor], topk: int, window: int,
                    softmax_scale: float = None, k_scale: float = 1.0, v_scale: float = 1.0,
                    workspace: Optional[torch.Tensor] = None):
    """Returns the workspace tensor so callers can reuse it across steps."""
    args, workspace, _keep = hys_decode_step_args(q_full, k_cache, v_cache, cache_len, o_full, token_scores, idx,
                                                  q_sparse, o_sparse, topk, window, softmax_scale, k_scale, v_scale,
                                                  workspace)
    check(_lib.load().hys_decode_step(*args))
    return workspace


def hys_decode_step_noalloc(q_full, k_cache, v_cache, cache_len: Sequence[int], o_full, token_scores, idx,
                            q_sparse: Sequence[torch.Tensor], o_sparse: Sequence[torch.Tensor], topk: int, window: int,
                            softmax_scale: float = None, k_scale: float = 1.0, v_scale: float = 1.0):
    """hys_decode_step on the library's fixed scratch array: no workspace is
    allocated by the call or by this wrapper."""
    lib = _lib.load()
    p = HysDecodeParams(softmax_scale or 1.0 / math.sqrt(q_full.shape[-1]), k_scale, v_scale, topk, window)
    lens = (ctypes.c_int64 * len(cache_len))(*[int(x) for x in cache_len])
    n = len(q_sparse)
    qs = (HysTensor4 * max(n, 1))(*[tensor4(t) for t in q_sparse])
    os_ = (HysTensor4 * max(n, 1))(*[tensor4(t) for t in o_sparse])
    check(lib.hys_decode_step_noalloc(ctypes.byref(p), tensor4(q_full), tensor4(k_cache), tensor4(v_cache), lens,
                                      tensor4(o_full), _ptr(token_scores), _ptr(idx), n, qs, os_,
                                      _stream(q_full.device)))


def hys_hysparse_decode_step(q_full, k_cache, v_cache, cache_len: Sequence[int], o_full, block_scores, idx,
                             q_sparse: Sequence[torch.Tensor], k_win_new: Sequence[torch.Tensor],
                             v_win_new: Sequence[torch.Tensor], k_ring: Sequence[torch.Tensor],
                             v_ring: Sequence[torch.Tensor], gate_w: Sequence[torch.Tensor],
                             o_sparse: Sequence[torch.Tensor], topk: int, softmax_scale: float = None,
                             workspace: Optional[torch.Tensor] = None):
    """One HySparse decode step; the rings are updated in place.  Returns the workspace for reuse."""
    lib = _lib.load()
    p = HysHsDecodeParams(softmax_scale or 1.0 / math.sqrt(q_full.shape[-1]), topk, 64)
    lens = (ctypes.c_int64 * len(cache_len))(*[int(x) for x in cache_len])
    n = len(q_sparse)

    def arr(ts):
        return (HysTensor4 * max(n, 1))(*[tensor4(t) for t in ts])
    gw = (ctypes.c_void_p * max(n, 1))(*[t.data_ptr() for t in gate_w])
    args = [ctypes.byref(p), tensor4(q_full), tensor4(k_cache), tensor4(v_cache), lens, tensor4(o_full),
            _ptr(block_scores), _ptr(idx), n, arr(q_sparse), arr(k_win_new), arr(v_win_new), arr(k_ring),
            arr(v_ring), gw, arr(o_sparse)]
    nb = ctypes.c_size_t(0)
    check(lib.hys_hysparse_decode_step(*args, None, ctypes.byref(nb), None))
    if workspace is None or workspace.numel() < nb.value:
        workspace = _workspace(nb.value, q_full.device)
    nb2 = ctypes.c_size_t(workspace.numel())
    check(lib.hys_hysparse_decode_step(*args, _ptr(workspace), ctypes.byref(nb2), _stream(q_full.device)))
    return workspace


def hys_kv_bridge_fwd(h, w_k, w_v, k_cache, v_cache, k_scale: float, v_scale: float,
                      amax: Optional[torch.Tensor] = None):
    """KV Bridging into the fp8 cache.  h: [B, L, d_model] (or [B, L, 1, d_model]) bf16;
    w_k, w_v: [Hkv*D, d_model] bf16 contiguous; k_cache, v_cache: [B, L, Hkv, D] fp8 (uint8 or
    float8_e4m3fn); amax: 2 fp32 (max |K|, max |V|) or None."""
    lib = _lib.load()
    h4 = h.unsqueeze(2) if h.dim() == 3 else h
    if not (w_k.is_contiguous() and w_v.is_contiguous()):
        raise ValueError("w_k and w_v must be contiguous [Hkv*D, d_model]")
    p = HysBridgeParams(k_scale, v_scale)
    check(lib.hys_kv_bridge_fwd(ctypes.byref(p), tensor4(h4), _ptr(w_k), _ptr(w_v), tensor4(k_cache),
                                tensor4(v_cache), _ptr(amax), _stream(h.device)))


def hys_window_attn_fwd(q, k_win, v_win, window: int, o, lse=None, softmax_scale: float = None, k_scale: float = 1.0,
                        v_scale: float = 1.0):
    """The window branch alone (no gate): o and its natural-log lse [B, Hq, L]."""
    lib = _lib.load()
    p = HysAttnParams(softmax_scale or 1.0 / math.sqrt(q.shape[-1]), k_scale, v_scale)
    check(lib.hys_window_attn_fwd(ctypes.byref(p), tensor4(q), tensor4(k_win), tensor4(v_win), window, tensor4(o),
                                  _ptr(lse), _stream(q.device)))


def hys_full_attn_bwd(q, k, v, o, lse, d_o, dq, dk, dv, accumulate_kv: bool = False, softmax_scale: float = None):
    """Gradients of the full layer's causal attention: dq (fp32) overwritten; dk, dv (fp32) overwritten or,
    with accumulate_kv, added to."""
    lib = _lib.load()
    p = HysAttnParams(softmax_scale or 1.0 / math.sqrt(q.shape[-1]), 1.0, 1.0)
    args = [ctypes.byref(p), tensor4(q), tensor4(k), tensor4(v), tensor4(o), _ptr(lse), tensor4(d_o), tensor4(dq),
            tensor4(dk), tensor4(dv), int(bool(accumulate_kv))]
    nb = ctypes.c_size_t(0)
    check(lib.hys_full_attn_bwd(*args, None, ctypes.byref(nb), None))
    ws = _workspace(nb.value, q.device)
    nb = ctypes.c_size_t(ws.numel())
    check(lib.hys_full_attn_bwd(*args, _ptr(ws), ctypes.byref(nb), _stream(q.device)))
    return ws


def hys_sparse_layer_bwd(q, k, v, idx, k_win, v_win, window: int, gate_w, o_sparse, lse_sparse, o_win, lse_win, d_o,
                         dq, dk, dv, dk_win, dv_win, dgate_w, accumulate_kv: bool = False, gate_b=None,
                         topk: int = None, softmax_scale: float = None, dgate_b=None):
    """Gradients of one HySparse sparse layer.  idx: [B, L, topk] block ids, or [Hkv, B, L, topk] per KV group.
    dgate_b: [Hq] fp32 for the gate bias's gradient, or None."""
    lib = _lib.load()
    p = HysAttnParams(softmax_scale or 1.0 / math.sqrt(q.shape[-1]), 1.0, 1.0)
    kk = idx.shape[-1] if topk is None else topk
    gs, ib = (idx.stride(0), idx[0]) if idx.dim() == 4 else (0, idx)
    sp = HysSparseParams(64, kk, 1, 0, ib.stride(0), ib.stride(1), gs)
    args = [ctypes.byref(p), tensor4(q), tensor4(k), tensor4(v), ctypes.byref(sp), _ptr(idx), tensor4(k_win),
            tensor4(v_win), window, _ptr(gate_w), _ptr(gate_b), tensor4(o_sparse), _ptr(lse_sparse), tensor4(o_win),
            _ptr(lse_win), tensor4(d_o), tensor4(dq), tensor4(dk), tensor4(dv), int(bool(accumulate_kv)),
            tensor4(dk_win), tensor4(dv_win), _ptr(dgate_w), _ptr(dgate_b)]
    nb = ctypes.c_size_t(0)
    check(lib.hys_sparse_layer_bwd(*args, None, ctypes.byref(nb), None))
    ws = _workspace(nb.value, q.device)
    nb = ctypes.c_size_t(ws.numel())
    check(lib.hys_sparse_layer_bwd(*args, _ptr(ws), ctypes.byref(nb), _stream(q.device)))
    return ws


def abi_version() -> int:
    return _lib.load().hys_abi_version()
