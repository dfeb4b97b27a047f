"""HySparse / HySparse2 hybrid-block attention for AMD MI355X (gfx950).

The compute lives in libhys.so (hand-written HIP kernels behind a C ABI,
declared in include/hys.h).  This package holds the ctypes binding (`ops`),
the hybrid-block sequencing of those calls (`block`) and the build script.
"""
from .ops import (abi_version, hys_decode_step, hys_full_attn_fwd, hys_hysparse_decode_step,  # noqa: F401
                  hys_kv_bridge_fwd, hys_select_topk, hys_sparse_attn_fwd, hys_sparse_layer_fwd, hys_swa_gate_fwd, tensor4)
