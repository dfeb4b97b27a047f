"""ctypes view of libhys.so (the C ABI declared in include/hys.h).

Loading fails loudly when the library has not been built: there is no
fallback implementation of any operation.
"""
import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libhys.so")

HYS_OK = 0
HYS_F32, HYS_BF16, HYS_FP8_E4M3 = 0, 1, 2
HYS_SCORE_NONE, HYS_SCORE_BLOCK, HYS_SCORE_TILE_TOKEN, HYS_SCORE_BLOCK_GROUP = 0, 1, 2, 3

# every symbol include/hys.h declares
EXPORTED = (
    "hys_full_attn_fwd", "hys_select_topk", "hys_sparse_attn_fwd", "hys_swa_gate_fwd",
    "hys_decode_step", "hys_decode_step_noalloc", "hys_sparse_layer_fwd", "hys_kv_bridge_fwd", "hys_hysparse_decode_step",
    "hys_select_topk_blocks", "hys_window_attn_fwd", "hys_full_attn_bwd", "hys_sparse_layer_bwd",
    "hys_last_error", "hys_status_string", "hys_abi_version",
)


class HysTensor4(ctypes.Structure):
    _fields_ = [("ptr", ctypes.c_void_p), ("dtype", ctypes.c_int32),
                ("shape", ctypes.c_int64 * 4), ("stride", ctypes.c_int64 * 4)]


class HysAttnParams(ctypes.Structure):
    _fields_ = [("softmax_scale", ctypes.c_float), ("k_scale", ctypes.c_float), ("v_scale", ctypes.c_float),
                ("causal", ctypes.c_int32), ("q_offset", ctypes.c_int64)]

    def __init__(self, softmax_scale=0.0, k_scale=1.0, v_scale=1.0, causal=1, q_offset=0):
        super().__init__(softmax_scale, k_scale, v_scale, causal, q_offset)


class HysScoreParams(ctypes.Structure):
    _fields_ = [("mode", ctypes.c_int32), ("size", ctypes.c_int32)]


class HysSparseParams(ctypes.Structure):
    _fields_ = [("granularity", ctypes.c_int32), ("k", ctypes.c_int32), ("q_tile", ctypes.c_int32),
                ("forced_window", ctypes.c_int32), ("idx_batch_stride", ctypes.c_int64),
                ("idx_row_stride", ctypes.c_int64), ("idx_group_stride", ctypes.c_int64)]


class HysDecodeParams(ctypes.Structure):
    _fields_ = [("softmax_scale", ctypes.c_float), ("k_scale", ctypes.c_float), ("v_scale", ctypes.c_float),
                ("topk", ctypes.c_int32), ("window", ctypes.c_int32)]


class HysHsDecodeParams(ctypes.Structure):
    _fields_ = [("softmax_scale", ctypes.c_float), ("topk", ctypes.c_int32), ("block", ctypes.c_int32)]


class HysBridgeParams(ctypes.Structure):
    _fields_ = [("k_scale", ctypes.c_float), ("v_scale", ctypes.c_float)]


_lib = None


def load(path: str = LIB_PATH):
    """Load libhys.so once; raise if it is missing or incomplete."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(
            f"libhys.so not found at {path}: build it first "
            "(python -c 'import __graft_entry__ as g; g.build()' or python hybrid_sparse_attention_flash_amd/build.py)")
    lib = ctypes.CDLL(path)
    for name in EXPORTED:
        if not hasattr(lib, name):
            raise RuntimeError(f"libhys.so lacks symbol {name}")
    T4 = HysTensor4
    P = ctypes.POINTER
    vp, sz = ctypes.c_void_p, ctypes.c_size_t
    lib.hys_full_attn_fwd.argtypes = [P(HysAttnParams), T4, T4, T4, T4, vp, P(HysScoreParams), vp, vp, P(sz), vp]
    lib.hys_select_topk.argtypes = [vp, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int32, vp, vp, vp,
                                    P(sz), vp]
    lib.hys_sparse_attn_fwd.argtypes = [P(HysAttnParams), T4, T4, T4, P(HysSparseParams), vp, T4, vp, vp, P(sz), vp]
    lib.hys_swa_gate_fwd.argtypes = [P(HysAttnParams), T4, T4, T4, ctypes.c_int32, T4, vp, vp, vp, T4, vp]
    lib.hys_decode_step.argtypes = [P(HysDecodeParams), T4, T4, T4, P(ctypes.c_int64), T4, vp, vp, ctypes.c_int32,
                                    P(T4), P(T4), vp, P(sz), vp]
    lib.hys_decode_step_noalloc.argtypes = [P(HysDecodeParams), T4, T4, T4, P(ctypes.c_int64), T4, vp, vp,
                                            ctypes.c_int32, P(T4), P(T4), vp]
    lib.hys_sparse_layer_fwd.argtypes = [P(HysAttnParams), T4, T4, T4, P(HysSparseParams), vp, T4, T4,
                                         ctypes.c_int32, vp, vp, T4, vp]
    lib.hys_kv_bridge_fwd.argtypes = [P(HysBridgeParams), T4, vp, vp, T4, T4, vp, vp]
    lib.hys_select_topk_blocks.argtypes = [vp, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int32,
                                           ctypes.c_int32, vp, vp, P(sz), vp]
    lib.hys_hysparse_decode_step.argtypes = [P(HysHsDecodeParams), T4, T4, T4, P(ctypes.c_int64), T4, vp, vp,
                                             ctypes.c_int32, P(T4), P(T4), P(T4), P(T4), P(T4), P(vp), P(T4), vp,
                                             P(sz), vp]
    lib.hys_window_attn_fwd.argtypes = [P(HysAttnParams), T4, T4, T4, ctypes.c_int32, T4, vp, vp]
    lib.hys_full_attn_bwd.argtypes = [P(HysAttnParams), T4, T4, T4, T4, vp, T4, T4, T4, T4, ctypes.c_int32, vp,
                                      P(sz), vp]
    lib.hys_sparse_layer_bwd.argtypes = [P(HysAttnParams), T4, T4, T4, P(HysSparseParams), vp, T4, T4,
                                         ctypes.c_int32, vp, vp, T4, vp, T4, vp, T4, T4, T4, T4, ctypes.c_int32, T4,
                                         T4, vp, vp, vp, P(sz), vp]
    for name in ("hys_full_attn_fwd", "hys_select_topk", "hys_sparse_attn_fwd", "hys_swa_gate_fwd",
                 "hys_decode_step", "hys_decode_step_noalloc", "hys_sparse_layer_fwd", "hys_kv_bridge_fwd", "hys_hysparse_decode_step",
                 "hys_select_topk_blocks", "hys_window_attn_fwd", "hys_full_attn_bwd", "hys_sparse_layer_bwd"):
        getattr(lib, name).restype = ctypes.c_int
    lib.hys_last_error.restype = ctypes.c_char_p
    lib.hys_last_error.argtypes = []
    lib.hys_status_string.restype = ctypes.c_char_p
    lib.hys_status_string.argtypes = [ctypes.c_int]
    lib.hys_abi_version.restype = ctypes.c_int
    lib.hys_abi_version.argtypes = []
    _lib = lib
    return lib


class HysError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{load().hys_status_string(status).decode()}: {message}")
        self.status = status


def check(status: int):
    if status != HYS_OK:
        raise HysError(status, load().hys_last_error().decode())
