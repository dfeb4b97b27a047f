"""KV Bridging: the cross-decoder full layer's K/V projected from hidden states
and written into the shared fp8 MQA cache.

TEST INFRASTRUCTURE ONLY (see the package header).

The HySparse2 pages describe KV Bridging (airebao HySparse2 news, outer "KV
Bridging" paragraph; demingchina commentary, section 02): the full-attention
layers of the cross-decoder no longer project their K/V from their own input
but from the hidden states of the self-decoder's full-attention layer, so the
KV is materialised once; the cache is MQA (one KV head per layer group, MQA
paragraph) and sized in FP8 (key-data table).  They give no widths, no
projection form beyond "projected", and no quantisation rule.  Readings taken
here (listed with the others in the design notes):

  * projection: K[b,t,:] = h[b,t,:] @ W_k^T and V[b,t,:] = h[b,t,:] @ W_v^T,
    no bias, W_k, W_v of shape [Hkv*D, d_model] (the usual [out, in] layout);
  * quantisation: one fp32 scale per cache tensor (the same per-tensor scale
    the attention calls dequantise with), code = e4m3(x * (1/s)) rounded to
    nearest-even and saturated at +-448, the largest finite e4m3fn value (a
    NaN written into a shared cache would poison every later attention);
  * the call also reports max |K| and max |V| so that a caller can set the
    next scale (s = amax / 448).

Precision rule for the codes: where floating point decides an integer the
oracle takes the decision in the kernel's precision, so the exact (float64)
dot product is rounded to fp32 before the fp32 multiply by the fp32 reciprocal
of the scale, and only then encoded.
"""
import numpy as np

from .fp8 import E4M3_MAX

E4M3_MIN_NORMAL_EXP = -6      # 2^-6: smallest normal magnitude
E4M3_SUB_STEP = 2.0 ** -9     # spacing of the subnormals (and of [2^-6, 2^-5))


def _round_half_even(x: np.ndarray) -> np.ndarray:
    """Round-half-to-even of exactly represented float64 values."""
    return np.rint(x)   # numpy's rint rounds halves to even


def encode_e4m3(x) -> np.ndarray:
    """float32/float64 values -> OCP e4m3fn codes (uint8), from the format.

    Round to the nearest representable value, ties to the even mantissa;
    magnitudes that round above 448 saturate to 448 (S.1111.110); NaN maps to
    the NaN code S.1111.111.  Inputs are exact in float64, and every step below
    (scaling by powers of two, rounding an exact value) is exact.
    """
    x = np.asarray(x, dtype=np.float64)
    sign = np.signbit(x).astype(np.uint8) << 7
    a = np.abs(x)
    codes = np.zeros(x.shape, dtype=np.uint8)
    nan = np.isnan(x)
    sub = a < 2.0 ** E4M3_MIN_NORMAL_EXP
    # subnormal range: multiples of 2^-9 (m = 8 becomes the smallest normal 2^-6, code 0x08)
    m_sub = _round_half_even(np.where(sub, a, 0.0) / E4M3_SUB_STEP).astype(np.int64)
    codes = np.where(sub, m_sub.astype(np.uint8), codes)
    # normal range: 1.m * 2^e, m in eighths
    with np.errstate(divide="ignore", invalid="ignore"):
        e = np.floor(np.log2(np.where(sub | nan, 1.0, a))).astype(np.int64)
    # log2 of an exact value can land one off at power-of-two edges; fix it up
    e = np.where(np.ldexp(1.0, e) > a, e - 1, e)
    e = np.where(np.ldexp(1.0, e + 1) <= a, e + 1, e)
    frac = np.ldexp(np.where(sub | nan, 1.0, a), -e) - 1.0          # in [0, 1)
    m = _round_half_even(frac * 8.0).astype(np.int64)
    carry = m == 8
    e = np.where(carry, e + 1, e)
    m = np.where(carry, 0, m)
    field = e + 7
    over = (field > 15) | ((field == 15) & (m > 6))
    field = np.where(over, 15, field)
    m = np.where(over, 6, m)
    normal = ((field << 3) | m).astype(np.uint8)
    codes = np.where(~sub & ~nan, normal, codes)
    codes = np.where(nan, np.uint8(0x7F), codes)
    return (codes | sign).astype(np.uint8)


def quantize_kernel_precision(x: np.ndarray, scale: float) -> np.ndarray:
    """Codes for exact values x under the kernel's fp32 steps (see the header)."""
    inv = np.float32(1.0) / np.float32(scale)
    y = np.asarray(x, dtype=np.float64).astype(np.float32) * inv
    return encode_e4m3(y.astype(np.float64))


def kv_bridge(h: np.ndarray, w_k: np.ndarray, w_v: np.ndarray, k_scale: float, v_scale: float):
    """Project and quantise one layer's bridged K/V.

    h [B, L, d_model], w_k / w_v [Hkv*D, d_model] (float64 holding the bf16
    values).  Returns (k_codes, v_codes, k_exact, v_exact, amax_k, amax_v) with
    codes [B, L, Hkv*D] uint8 and the exact float64 projections beside them.
    """
    h = np.asarray(h, dtype=np.float64)
    k = h @ np.asarray(w_k, dtype=np.float64).T
    v = h @ np.asarray(w_v, dtype=np.float64).T
    return (quantize_kernel_precision(k, k_scale), quantize_kernel_precision(v, v_scale), k, v,
            float(np.max(np.abs(k))) if k.size else 0.0, float(np.max(np.abs(v))) if v.size else 0.0)


assert E4M3_MAX == 448.0
