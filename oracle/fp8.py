"""OCP FP8 E4M3 (e4m3fn) decoding, built from the format definition.

TEST INFRASTRUCTURE ONLY (see the package header).

The HySparse2 pages size the 1M-token KV cache in FP8 (airebao HySparse2 news,
key-data table; demingchina commentary, section 05); they do not name the
FP8 variant.  The reading taken here is OCP E4M3 "fn": 1 sign bit, 4 exponent
bits with bias 7, 3 mantissa bits, subnormals when the exponent field is 0,
no infinities, and S.1111.111 as the only NaN pattern (so the largest finite
magnitude is 1.75 * 2^8 = 448).  A stored element's value is decode(byte) * s
with one fp32 scale s per tensor.
"""
import numpy as np

E4M3_BIAS = 7
E4M3_MAX = 448.0


def decode_byte(b: int) -> float:
    """Value of one e4m3fn encoding, straight from the bit fields."""
    b = int(b) & 0xFF
    sign = -1.0 if (b >> 7) & 1 else 1.0
    e = (b >> 3) & 0xF
    m = b & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return sign * (m / 8.0) * 2.0 ** (1 - E4M3_BIAS)
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - E4M3_BIAS)


def decode_table() -> np.ndarray:
    """All 256 encodings decoded to float64."""
    return np.array([decode_byte(b) for b in range(256)], dtype=np.float64)


_TABLE = decode_table()


def dequantize(codes: np.ndarray, scale: float) -> np.ndarray:
    """fp8 codes (uint8 array) -> float64 values decode(code) * scale."""
    codes = np.asarray(codes, dtype=np.uint8)
    return _TABLE[codes] * float(scale)
