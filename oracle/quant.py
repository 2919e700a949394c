"""FP8 (OCP E4M3) and INT8 KV-cache quantization, as plain NumPy.

Test infrastructure only (see the package docstring).

The pages name the idea -- store K/V in INT8/FP8 and keep higher-precision
arithmetic -- without a format or a scaling rule (page "KV Cache and Inference
Optimization", section "KV quantization"). This reference fixes the plainest
reading, stated in full so that both sides take every rounding decision in the
same precision:

  * format: OCP 8-bit floating point E4M3 -- 1 sign bit, 4 exponent bits (bias
    7), 3 mantissa bits; exponent field 0 encodes subnormals 2^-6 * m/8; no
    infinities; S.1111.111 is NaN; the largest finite magnitude is 448;
  * one scale per token row of one KV head (D values): scale = amax / 448 in
    float32, inv = 448 / amax in float32 (amax = 0 gives scale 1 and inv 1);
  * code = nearest E4M3 value to float32(x * inv), ties to the even code,
    magnitudes above 448 saturate to 448, the sign bit is kept (a negative
    value that rounds to zero gives -0);
  * the cached value a kernel attends over is decode(code) * scale (exact in
    float64).

INT8 (the page's other named option) follows the same rule with 127 as the
largest code: scale = amax / 127, inv = 127 / amax (float32; amax = 0 gives 1
and 1), code = float32(x * inv) rounded to the nearest integer (ties to even),
clamped to [-127, 127]; the value is code * scale.

A row holding a NaN or an infinity has no finite scale. The pages say nothing
about such rows; the reading here is that the whole row becomes unreadable:
scale NaN and every code set to the format's marker -- E4M3 0x7F (its NaN),
INT8 -128 (the one code a finite row never gets) -- so every value of the row
reads back as NaN, as a NaN in a 16-bit cache would make the attention NaN.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0


def e4m3_value(code: int) -> float:
    """Real value of one E4M3 code (NaN for S.1111.111)."""
    code = int(code) & 0xFF
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return sign * 2.0 ** -6 * (m / 8.0)
    return sign * 2.0 ** (e - 7) * (1.0 + m / 8.0)


# every non-negative finite code and its value, in increasing order (codes 0..126)
_POS_CODES = np.arange(0, 0x7F, dtype=np.int64)
_POS_VALUES = np.array([e4m3_value(c) for c in _POS_CODES], dtype=np.float64)
assert np.all(np.diff(_POS_VALUES) > 0)


# the value of every code, from e4m3_value (built once: decoding looks codes up)
_E4M3_TABLE = np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """float64 values of uint8 codes."""
    return _E4M3_TABLE[np.asarray(codes, dtype=np.uint8)]


def e4m3_encode(x: np.ndarray) -> np.ndarray:
    """Nearest E4M3 code (ties to the even code), saturating at 448; NaN -> 0x7F."""
    x = np.asarray(x, dtype=np.float64)
    a = np.minimum(np.abs(x), E4M3_MAX)
    hi = np.clip(np.searchsorted(_POS_VALUES, a, side="left"), 0, len(_POS_VALUES) - 1)
    lo = np.maximum(hi - 1, 0)
    d_hi = np.abs(_POS_VALUES[hi] - a)
    d_lo = np.abs(a - _POS_VALUES[lo])
    pick_lo = (d_lo < d_hi) | ((d_lo == d_hi) & (_POS_CODES[lo] % 2 == 0))
    code = np.where(pick_lo, _POS_CODES[lo], _POS_CODES[hi]).astype(np.uint8)
    code = np.where(np.signbit(x), code | 0x80, code).astype(np.uint8)  # the sign is kept, zero included
    code = np.where(np.isnan(x), np.uint8(0x7F), code).astype(np.uint8)
    return code


def quantize_rows(x: np.ndarray):
    """Quantize the last axis of float32 ``x`` row by row.

    Returns (codes uint8 with x's shape, scales float32 with x's shape minus the
    last axis), following the module docstring step by step in float32.
    """
    x = np.asarray(x, dtype=np.float32)
    amax = np.max(np.abs(x), axis=-1).astype(np.float32)  # NaN if the row holds one
    bad = ~np.isfinite(amax)
    zero = amax == 0
    safe = np.where(zero | bad, np.float32(1), amax).astype(np.float32)
    scale = np.where(zero, np.float32(1), safe / np.float32(E4M3_MAX)).astype(np.float32)
    inv = np.where(zero, np.float32(1), np.float32(E4M3_MAX) / safe).astype(np.float32)
    y = (np.where(bad[..., None], np.float32(0), x) * inv[..., None]).astype(np.float32)
    codes = np.where(bad[..., None], np.uint8(0x7F), e4m3_encode(y)).astype(np.uint8)
    return codes, np.where(bad, np.float32(np.nan), scale).astype(np.float32)


def dequantize_rows(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """float64 values decode(code) * scale."""
    return e4m3_decode(codes) * np.asarray(scales, dtype=np.float64)[..., None]


INT8_MAX = 127.0


def quantize_rows_int8(x: np.ndarray):
    """INT8 codes (int8, x's shape) and float32 scales of the last axis of ``x``,
    following the module docstring step by step in float32."""
    x = np.asarray(x, dtype=np.float32)
    amax = np.max(np.abs(x), axis=-1).astype(np.float32)  # NaN if the row holds one
    bad = ~np.isfinite(amax)
    zero = amax == 0
    safe = np.where(zero | bad, np.float32(1), amax).astype(np.float32)
    scale = np.where(zero, np.float32(1), safe / np.float32(INT8_MAX)).astype(np.float32)
    inv = np.where(zero, np.float32(1), np.float32(INT8_MAX) / safe).astype(np.float32)
    y = (np.where(bad[..., None], np.float32(0), x) * inv[..., None]).astype(np.float32)
    codes = np.clip(np.rint(y.astype(np.float64)), -INT8_MAX, INT8_MAX).astype(np.int8)
    codes = np.where(bad[..., None], np.int8(-128), codes).astype(np.int8)
    return codes, np.where(bad, np.float32(np.nan), scale).astype(np.float32)


def int8_decode(codes: np.ndarray) -> np.ndarray:
    """float64 values of int8 codes stored as raw bytes (uint8) or int8."""
    return np.asarray(codes).view(np.int8).astype(np.float64) if np.asarray(codes).dtype == np.uint8 \
        else np.asarray(codes, dtype=np.int8).astype(np.float64)


def decode_codes(codes: np.ndarray, fmt: str) -> np.ndarray:
    """float64 values of 8-bit codes in format ``fmt`` ("e4m3" or "int8")."""
    if fmt == "e4m3":
        return e4m3_decode(codes)
    if fmt == "int8":
        return int8_decode(codes)
    raise ValueError(f"unknown code format {fmt!r}")


def quantize_rows_fmt(x: np.ndarray, fmt: str):
    """(codes as raw uint8 bytes, float32 scales) in format ``fmt``."""
    if fmt == "e4m3":
        return quantize_rows(x)
    if fmt == "int8":
        c, s = quantize_rows_int8(x)
        return c.view(np.uint8), s
    raise ValueError(f"unknown code format {fmt!r}")
