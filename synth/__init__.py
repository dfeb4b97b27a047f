"""Seeded synthetic inputs and workload shapes for the HySparse / HySparse2 hot path.

This module is shared by the CPU oracle, the tests, the benchmark and the
smoke entry point.  It holds no arithmetic of the attention method itself:
only the workload shapes, seeded normal draws, and the one-time storage
conversions (fp32 -> bf16 round-to-nearest-even, fp32 -> fp8 e4m3fn with a
per-tensor scale) that produce the exact bytes both sides consume.

Random streams: every tensor is drawn from
``numpy.random.default_rng([seed, cfg_id, crc32(tag)])`` so streams are
independent of generation order and reproducible on any host.
"""
from __future__ import annotations

import dataclasses
import zlib
from dataclasses import dataclass, field
from typing import Dict, List, Optional

import numpy as np
import torch

FP8_E4M3_MAX = 448.0


@dataclass(frozen=True)
class Workload:
    """Shape and structure of one hybrid-block workload.

    variant: 'hysparse'  - block-level selection + gated sliding-window branch
             'hysparse2' - token-level selection + forced recent window
             'decode'    - HySparse2 single-token decode against a long cache
    """
    name: str
    cfg_id: int
    B: int
    L: int            # sequence length (decode: cache length N)
    Hq: int
    Hkv: int
    D: int
    q_dtype: str      # 'f32' | 'bf16'
    kv_dtype: str     # 'f32' | 'bf16' | 'fp8'
    n_sparse: int
    variant: str
    block: int = 64   # key-block size (HySparse) / query-tile size (HySparse2)
    topk: int = 16
    window: int = 128
    needles: int = 0
    needle_scale: float = 4.0
    gate_std: float = 0.02
    cache_lens: Optional[tuple] = None   # decode only: per-sequence valid length

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    @property
    def scale(self) -> float:
        return 1.0 / float(np.sqrt(self.D))

    @property
    def nblk(self) -> int:
        return (self.L + self.block - 1) // self.block

    def lens(self) -> List[int]:
        if self.cache_lens is not None:
            return list(self.cache_lens)
        return [self.L] * self.B

    def shrink(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)

    def as_dict(self) -> Dict:
        d = dataclasses.asdict(self)
        d["cache_lens"] = list(self.cache_lens) if self.cache_lens else None
        return d


# The five workloads of the hot path.  Shapes follow the HySparse pages: 64-token
# blocks and a 128-token window (QbitAI article, method section; TechWalker
# write-up, method section), 1:3 and 1:11 hybrid ratios (TechWalker write-up,
# model setup), token-level top-1024 plus a recent-128 window over one shared
# MQA FP8 KV cache (airebao HySparse2 news, token-level selection / forced window /
# MQA paragraphs), and 1M-token decode (airebao HySparse2 news, key-data table).
WORKLOADS: Dict[str, Workload] = {
    "tiny_fp32": Workload(
        name="tiny_fp32", cfg_id=1, B=1, L=1024, Hq=8, Hkv=1, D=64,
        q_dtype="f32", kv_dtype="f32", n_sparse=3, variant="hysparse",
        block=64, topk=4, window=128),
    "dense7b_16k": Workload(
        name="dense7b_16k", cfg_id=2, B=1, L=16384, Hq=32, Hkv=8, D=128,
        q_dtype="bf16", kv_dtype="bf16", n_sparse=3, variant="hysparse",
        block=64, topk=16, window=128),
    "moe80b_32k": Workload(
        name="moe80b_32k", cfg_id=3, B=1, L=32768, Hq=32, Hkv=4, D=128,
        q_dtype="bf16", kv_dtype="bf16", n_sparse=11, variant="hysparse",
        block=64, topk=16, window=128, needles=32, needle_scale=4.0),
    "hysparse2_64k": Workload(
        name="hysparse2_64k", cfg_id=4, B=1, L=65536, Hq=64, Hkv=1, D=128,
        q_dtype="bf16", kv_dtype="fp8", n_sparse=3, variant="hysparse2",
        block=64, topk=1024, window=128),
    "decode_1m": Workload(
        name="decode_1m", cfg_id=5, B=4, L=1048576, Hq=64, Hkv=1, D=128,
        q_dtype="bf16", kv_dtype="fp8", n_sparse=11, variant="decode",
        block=64, topk=1024, window=128),
}

WORKLOAD_ORDER = ["tiny_fp32", "dense7b_16k", "moe80b_32k", "hysparse2_64k", "decode_1m"]

# HySparse (block-level) decode: the 80B-like block's attention (32 query /
# 4 KV heads, bf16, 11 sparse layers, top-16 of 64-token blocks, window 128)
# one token at a time against a 128k-token cache per sequence.  The pages give
# no HySparse decode configuration; 128k x 4 sequences is the same KV byte
# count as the 1M-token fp8 HySparse2 decode workload.
HS_DECODE_WORKLOAD = Workload(
    name="hysparse_decode_128k", cfg_id=7, B=4, L=131072, Hq=32, Hkv=4, D=128,
    q_dtype="bf16", kv_dtype="bf16", n_sparse=11, variant="hsdecode",
    block=64, topk=16, window=128)


# ----------------------------------------------------------------------------
# seeded draws and storage conversions
# ----------------------------------------------------------------------------

def rng_for(seed: int, cfg_id: int, tag: str) -> np.random.Generator:
    return np.random.default_rng([int(seed), int(cfg_id), zlib.crc32(tag.encode())])


def normal(seed: int, cfg_id: int, tag: str, shape, std: float = 1.0) -> np.ndarray:
    x = rng_for(seed, cfg_id, tag).standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return x


def to_bf16(x: np.ndarray) -> torch.Tensor:
    """fp32 -> bf16, round to nearest even (torch's conversion), CPU tensor."""
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)


def to_fp8_e4m3(x: np.ndarray):
    """fp32 -> OCP fp8 e4m3fn bytes with one per-tensor scale s = amax/448.

    Returns (uint8 CPU tensor of encodings, float scale).  The stored value of
    element e is decode(byte_e) * s.
    """
    amax = float(np.abs(x).max()) if x.size else 1.0
    if amax == 0.0:
        amax = 1.0
    s = float(np.float32(amax / FP8_E4M3_MAX))
    y = np.clip(x / np.float32(s), -FP8_E4M3_MAX, FP8_E4M3_MAX).astype(np.float32)
    t = torch.from_numpy(np.ascontiguousarray(y)).to(torch.float8_e4m3fn).view(torch.uint8)
    b = t.numpy()
    if ((b & 0x7F) == 0x7F).any():
        raise ValueError("fp8 quantisation produced NaN encodings")
    return t, s


def store(x: np.ndarray, dtype: str):
    """Convert an fp32 draw to the workload's storage type.

    Returns (tensor, scale) where scale is 1.0 except for fp8.
    """
    if dtype == "f32":
        return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)), 1.0
    if dtype == "bf16":
        return to_bf16(x), 1.0
    if dtype == "fp8":
        return to_fp8_e4m3(x)
    raise ValueError(dtype)


# ----------------------------------------------------------------------------
# per-workload tensors (generated one at a time so large workloads stream)
# ----------------------------------------------------------------------------

def needle_positions(w: Workload, seed: int = 0) -> np.ndarray:
    if w.needles <= 0:
        return np.zeros(0, dtype=np.int64)
    r = rng_for(seed, w.cfg_id, "needles")
    return np.sort(r.choice(w.L, size=min(w.needles, w.L), replace=False)).astype(np.int64)


def gen_q(w: Workload, layer: int, seed: int = 0) -> torch.Tensor:
    """Query of layer `layer` (0 = the full-attention layer).

    Prefill: [B, L, Hq, D]; decode: [B, 1, Hq, D].
    """
    T = 1 if w.variant == "decode" else w.L
    x = normal(seed, w.cfg_id, f"q{layer}", (w.B, T, w.Hq, w.D))
    t, _ = store(x, w.q_dtype if w.q_dtype != "fp8" else "bf16")
    return t


def gen_kv(w: Workload, which: str, seed: int = 0):
    """Shared K or V of the hybrid block: [B, L, Hkv, D] in kv_dtype.

    Needles (when the workload has them) scale K at the needle positions,
    across all KV heads, before storage rounding; V is never scaled.
    Returns (tensor, scale).
    """
    assert which in ("k", "v")
    x = normal(seed, w.cfg_id, which, (w.B, w.L, w.Hkv, w.D))
    if which == "k" and w.needles > 0:
        pos = needle_positions(w, seed)
        x[:, pos, :, :] *= np.float32(w.needle_scale)
    return store(x, w.kv_dtype)


def gen_window_kv(w: Workload, layer: int, which: str, seed: int = 0):
    """Per-sparse-layer sliding-window K or V (HySparse only): [B, L, Hkv, D]."""
    assert which in ("kw", "vw") and layer >= 1
    x = normal(seed, w.cfg_id, f"{which}{layer}", (w.B, w.L, w.Hkv, w.D))
    return store(x, w.kv_dtype if w.kv_dtype != "fp8" else "bf16")


def gen_gate_w(w: Workload, layer: int, seed: int = 0) -> torch.Tensor:
    """Per-sparse-layer gate weights [Hq, D], fp32, N(0, gate_std^2)."""
    x = normal(seed, w.cfg_id, f"gate{layer}", (w.Hq, w.D), std=w.gate_std)
    return torch.from_numpy(x)


def gen_grad_out(w: Workload, layer: int, seed: int = 0) -> torch.Tensor:
    """Upstream gradient of layer `layer`'s output (0 = the full layer) for the
    backward pass: [B, L, Hq, D] bf16, N(0, 1)."""
    x = normal(seed, w.cfg_id, f"dout{layer}", (w.B, w.L, w.Hq, w.D))
    return to_bf16(x)


def to_f64(t: torch.Tensor) -> np.ndarray:
    """Exact upcast of a stored fp32 / bf16 tensor to float64 numpy.

    fp8 byte tensors are not handled here: each consumer decodes them itself.
    """
    if t.dtype == torch.uint8:
        raise TypeError("fp8 bytes must be decoded by the consumer")
    return t.to(torch.float64).numpy()


# ----------------------------------------------------------------------------
# KV Bridging inputs (HySparse2): the self-decoder full layer's hidden states
# and the cross-decoder full layer's K/V projection weights
# ----------------------------------------------------------------------------

# The pages name no model width; 4096 is the hidden size taken for the 64k
# HySparse2 workload (one MQA KV head of dimension 128, as in hysparse2_64k).
BRIDGE_WORKLOAD = {"name": "kv_bridge_64k", "cfg_id": 6, "B": 1, "L": 65536, "d_model": 4096, "Hkv": 1, "D": 128}


def gen_bridge(seed: int, cfg_id: int, B: int, L: int, d_model: int, n_out: int,
               outlier_frac: float = 0.01, outlier_scale: float = 8.0):
    """Hidden states h [B, L, d_model] and weights w_k, w_v [n_out, d_model], bf16 CPU tensors.

    h ~ N(0, 1) with a fixed 1% of channels scaled by 8 (the few large
    channels of normalised transformer activations); weights ~ N(0, 1/d_model)
    so the projections have unit-order spread.
    """
    h = normal(seed, cfg_id, "bridge_h", (B, L, d_model))
    n_out_ch = max(1, int(round(d_model * outlier_frac)))
    cols = np.sort(rng_for(seed, cfg_id, "bridge_outliers").choice(d_model, size=n_out_ch, replace=False))
    h[..., cols] *= np.float32(outlier_scale)
    std = float(1.0 / np.sqrt(d_model))
    wk = normal(seed, cfg_id, "bridge_wk", (n_out, d_model), std=std)
    wv = normal(seed, cfg_id, "bridge_wv", (n_out, d_model), std=std)
    return to_bf16(h), to_bf16(wk), to_bf16(wv)


def gen_hs_decode(w: Workload, seed: int = 0) -> Dict:
    """Inputs of one HySparse decode step (bf16 CPU tensors, gate fp32).

    q_full [B,1,Hq,D]; the shared cache k, v [B,N,Hkv,D]; per sparse layer l:
    q [B,1,Hq,D], the new token's window K/V [B,1,Hkv,D], the ring
    [B,window,Hkv,D] (window K/V of the earlier tokens; every slot is drawn,
    including slots that hold no token yet) and gate_w [Hq,D] ~ N(0, gate_std^2).
    """
    B, N, Hq, Hkv, D, W = w.B, w.L, w.Hq, w.Hkv, w.D, w.window
    out = {
        "q_full": to_bf16(normal(seed, w.cfg_id, "hsd_q0", (B, 1, Hq, D))),
        "k": to_bf16(normal(seed, w.cfg_id, "hsd_k", (B, N, Hkv, D))),
        "v": to_bf16(normal(seed, w.cfg_id, "hsd_v", (B, N, Hkv, D))),
        "q": [], "k_new": [], "v_new": [], "k_ring": [], "v_ring": [], "gate_w": [],
    }
    for l in range(1, w.n_sparse + 1):
        out["q"].append(to_bf16(normal(seed, w.cfg_id, f"hsd_q{l}", (B, 1, Hq, D))))
        out["k_new"].append(to_bf16(normal(seed, w.cfg_id, f"hsd_kn{l}", (B, 1, Hkv, D))))
        out["v_new"].append(to_bf16(normal(seed, w.cfg_id, f"hsd_vn{l}", (B, 1, Hkv, D))))
        out["k_ring"].append(to_bf16(normal(seed, w.cfg_id, f"hsd_kr{l}", (B, W, Hkv, D))))
        out["v_ring"].append(to_bf16(normal(seed, w.cfg_id, f"hsd_vr{l}", (B, W, Hkv, D))))
        out["gate_w"].append(torch.from_numpy(normal(seed, w.cfg_id, f"hsd_gate{l}", (Hq, D), std=w.gate_std)))
    return out
