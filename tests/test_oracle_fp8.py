"""Pins for the oracle's fp8 (OCP E4M3) codec and per-token quantiser.

The pages define no quantised cache; these pin the oracle's fp8 helpers to
the OCP E4M3 definition (closed forms, exhaustive round trips, the tie rule)
and to the quantiser's stated properties, so that the GPU quantiser and the
fp8 decode path are compared against something other than themselves.
"""
import numpy as np
import pytest

from oracle import fp8


def test_e4m3_landmarks():
    v = fp8.VALUES
    assert v[0x00] == 0.0 and not np.signbit(v[0x00])
    assert v[0x80] == 0.0 and np.signbit(v[0x80])          # negative zero
    assert v[0x01] == 2.0 ** -9                             # smallest subnormal
    assert v[0x07] == 7 * 2.0 ** -9                         # largest subnormal
    assert v[0x08] == 2.0 ** -6                             # smallest normal
    assert v[0x38] == 1.0                                   # exponent field 7 = bias
    assert v[0x39] == 1.125
    assert v[0x7E] == 448.0 and v[0xFE] == -448.0           # largest finite
    assert np.isnan(v[0x7F]) and np.isnan(v[0xFF])          # the only NaNs
    assert np.isfinite(v).sum() == 254
    pos = v[:0x7F]
    assert np.all(np.diff(pos) > 0)                         # codes 0..126 increase
    assert np.array_equal(v[0x80:0xFF], -v[0x00:0x7F])     # sign bit


def test_e4m3_round_trip_and_ties():
    finite = np.array([c for c in range(256) if np.isfinite(fp8.VALUES[c])], np.uint8)
    assert np.array_equal(fp8.encode(fp8.VALUES[finite].astype(np.float32)), finite)
    # ties go to the even code
    assert fp8.encode(np.float32([1.0625]))[0] == 0x38      # 1.0 | 1.125 -> 1.0
    assert fp8.encode(np.float32([1.1875]))[0] == 0x3A      # 1.125 | 1.25 -> 1.25
    assert fp8.encode(np.float32([1.5 * 2.0 ** -9]))[0] == 0x02  # subnormal tie
    assert fp8.encode(np.float32([-1.0625]))[0] == 0xB8
    # just off a tie goes to the nearer value
    assert fp8.encode(np.nextafter(np.float32([1.0625]), np.float32(2)))[0] == 0x39
    assert fp8.encode(np.float32([440.0]))[0] == 0x7E       # 432 | 448 -> 448
    with pytest.raises(ValueError):
        fp8.encode(np.float32([449.0]))


def test_quantiser_properties():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((64, 576)).astype(np.float32)
    x[3] = 0.0                                               # all-zero row
    x[7, 100] = 50.0                                         # one large entry
    codes, scale = fp8.quantize_rows(x)
    assert codes.shape == x.shape and codes.dtype == np.uint8 and scale.dtype == np.float32
    amax = np.abs(x).max(axis=1)
    np.testing.assert_array_equal(scale, (amax / np.float32(448)).astype(np.float32))
    assert scale[3] == 0 and np.all(codes[3] == 0)
    # each row's largest magnitude lands on +-448 (code 0x7E / 0xFE)
    rows = [r for r in range(64) if r != 3]
    arg = np.abs(x[rows]).argmax(axis=1)
    assert np.all(codes[rows, arg] & 0x7F == 0x7E)
    # dequantised error: at most half a step of the e4m3 grid
    deq = fp8.dequantize(codes, scale)
    err = np.abs(deq - x)
    bound = np.maximum(np.abs(x) * 2.0 ** -4, scale[:, None].astype(np.float64) * 2.0 ** -10)
    assert np.all(err <= bound * (1 + 1e-6))
    # signs survive
    nz = x != 0
    assert np.all(np.sign(deq[nz]) == np.sign(x[nz]))


def test_query_quantiser_properties():
    # per-vector (last axis) form of the FP8-MFMA attention path
    rng = np.random.default_rng(9)
    q = rng.standard_normal((3, 5, 576)).astype(np.float32)
    q[1, 2] = 0.0                                            # an all-zero query
    q[2, 4, 17] = -40.0                                      # one large entry
    codes, sigma = fp8.quantize_query(q)
    assert codes.shape == q.shape and codes.dtype == np.uint8 and sigma.shape == (3, 5)
    amax = np.abs(q).max(axis=-1)
    np.testing.assert_array_equal(sigma, (amax / np.float32(448)).astype(np.float32))
    assert sigma[1, 2] == 0 and np.all(codes[1, 2] == 0)
    # each vector's largest magnitude lands on +-448 with its sign
    assert codes[2, 4, 17] == 0xFE
    for i in range(3):
        for j in range(5):
            if (i, j) != (1, 2):
                assert codes[i, j, np.abs(q[i, j]).argmax()] & 0x7F == 0x7E
    # dequantised error: at most half a step of the e4m3 grid (the fp32
    # product q * (448 / amax) is within one rounding of q / sigma)
    deq = fp8.decode(codes) * sigma[..., None].astype(np.float64)
    bound = np.maximum(np.abs(q) * 2.0 ** -4, sigma[..., None].astype(np.float64) * 2.0 ** -10)
    assert np.all(np.abs(deq - q) <= bound * (1 + 1e-5))
    assert np.all(np.sign(deq[q != 0]) == np.sign(q[q != 0]))


def test_query_quantiser_exact_grid():
    # values on the e4m3 grid times 2^-5 with a largest magnitude of 448 * 2^-5
    # (= 14): 448 / 14 = 32 exactly, so every product is a grid value and the
    # codes come back unchanged (a divide-instead-of-multiply or a wrong
    # constant would move them)
    rng = np.random.default_rng(10)
    finite = np.array([c for c in range(256) if np.isfinite(fp8.VALUES[c])], np.uint8)
    c = rng.choice(finite, size=576).astype(np.uint8)
    c[0] = 0x7E
    q = (fp8.VALUES[c] * 2.0 ** -5).astype(np.float32)
    codes, sigma = fp8.quantize_query(q)
    assert sigma == np.float32(14.0 / 448.0)
    # negative zero and zero both decode to 0: compare values, not bytes
    np.testing.assert_array_equal(fp8.VALUES[codes], fp8.VALUES[c])
