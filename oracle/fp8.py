"""OCP FP8 E4M3 codes and the per-token cache quantiser -- TEST INFRASTRUCTURE ONLY.

Only the test suite may import this module; the product library never does,
and this module imports nothing from it.

E4M3 as the OCP 8-bit floating-point specification defines it: 1 sign bit, 4
exponent bits (bias 7), 3 mantissa bits; exponent field 0 holds the
subnormals m * 2^-9; there are no infinities, and S.1111.111 is NaN, so the
largest finite magnitude is 1.75 * 2^8 = 448.

The quantiser is the form the library documents for its fp8 cache (the
reference pages define none): per 576-wide row, scale = max|x| / 448 in fp32,
and every code is the e4m3 value nearest to the fp32 quotient x / scale
clamped to [-448, 448], ties to the even code; an all-zero row gets scale 0
and zero codes.  Dequantised row = e4m3_value(code) * scale.

Everything here is plain numpy, written out from those definitions.
"""
from __future__ import annotations

import numpy as np

MAX_FINITE = 448.0


def e4m3_value(code: int) -> float:
    """Value of one E4M3 byte (the OCP definition, term by term)."""
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return sign * m * 2.0 ** -9          # subnormal: 0.m * 2^(1 - 7)
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


VALUES = np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)
_POS = VALUES[:0x7F]  # codes 0x00 .. 0x7E: the non-negative finite values, increasing


def decode(codes) -> np.ndarray:
    """E4M3 bytes -> fp64 values (exact)."""
    return VALUES[np.asarray(codes, dtype=np.uint8)]


def encode(q) -> np.ndarray:
    """fp32 values in [-448, 448] -> nearest E4M3 bytes, ties to the even code."""
    q = np.asarray(q, dtype=np.float32)
    if np.any(np.isnan(q)) or np.any(np.abs(q) > MAX_FINITE):
        raise ValueError("encode expects finite values in [-448, 448]")
    a = np.abs(q).astype(np.float64)
    hi = np.searchsorted(_POS, a, side="left")          # first code with value >= a
    hi = np.minimum(hi, 0x7E)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - _POS[lo]
    d_hi = _POS[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    mag = np.where(a == _POS[hi], hi, np.where(pick_hi, hi, lo)).astype(np.uint8)
    neg = np.signbit(q)
    return np.where(neg, mag | 0x80, mag).astype(np.uint8)


def quantize_rows(x):
    """Per-row quantiser.  x: array-like [..., 576] (bf16 values widened exactly).
    Returns (codes uint8 [..., 576], scale fp32 [...])."""
    if hasattr(x, "detach"):
        import torch
        x = x.detach().to(device="cpu", dtype=torch.float32).numpy()
    xf = np.asarray(x, dtype=np.float32)
    amax = np.max(np.abs(xf), axis=-1)
    scale = (amax / np.float32(MAX_FINITE)).astype(np.float32)
    safe = np.where(scale > 0, scale, np.float32(1.0)).astype(np.float32)
    q = np.where(scale[..., None] > 0, xf / safe[..., None], np.float32(0.0)).astype(np.float32)
    q = np.clip(q, -MAX_FINITE, MAX_FINITE).astype(np.float32)
    return encode(q), scale


def dequantize(codes, scale) -> np.ndarray:
    """fp64 rows: e4m3_value(codes) * scale (exact in fp64)."""
    return decode(codes) * np.asarray(scale, dtype=np.float64)[..., None]


def quantize_query(q):
    """Per-(row, head) query quantiser of the FP8-MFMA attention path (the
    library's form; the pages define none).  q: array-like [..., 576] (bf16
    values widened exactly).  Per vector, in fp32: amax = max|q|,
    sigma = amax / 448, inv = 448 / amax (0 when amax is 0), and every code is
    the e4m3 value nearest to clamp(q * inv, -448, 448), ties to the even
    code.  Returns (codes uint8 [..., 576], sigma fp32 [...]); the dequantised
    query is e4m3_value(code) * sigma."""
    if hasattr(q, "detach"):
        import torch
        q = q.detach().to(device="cpu", dtype=torch.float32).numpy()
    qf = np.asarray(q, dtype=np.float32)
    amax = np.max(np.abs(qf), axis=-1).astype(np.float32)
    sigma = (amax / np.float32(MAX_FINITE)).astype(np.float32)
    safe = np.where(amax > 0, amax, np.float32(1.0)).astype(np.float32)
    inv = np.where(amax > 0, np.float32(MAX_FINITE) / safe, np.float32(0.0)).astype(np.float32)
    x = (qf * inv[..., None]).astype(np.float32)
    x = np.clip(x, -MAX_FINITE, MAX_FINITE).astype(np.float32)
    return encode(x), sigma
