"""Pins of the oracle's FP8 (E4M3) KV-cache codec (oracle/fp8.py).

The encoder is checked against an independent brute-force search (nearest
finite code by absolute distance, ties to the even code, saturation at
448) over random values, every code, every midpoint between neighbouring
codes and the saturation and subnormal edges; the decoder against codes
worked out by hand from the format definition; the attention on an FP8 pool
against the same attention on a float64 pool holding the dequantised values.
"""
import math

import numpy as np
import pytest

import oracle

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


# (code, value) worked out from sign / exponent (bias 7) / 3-bit mantissa
HAND_CODES = [
    (0x00, 0.0),
    (0x01, 2.0 ** -9),              # smallest subnormal: 1/8 * 2^-6
    (0x07, 7 * 2.0 ** -9),          # largest subnormal
    (0x08, 2.0 ** -6),              # smallest normal
    (0x30, 0.5),                    # e = 6
    (0x38, 1.0),                    # e = 7 (the bias)
    (0x3C, 1.5),                    # m = 4
    (0x3F, 1.875),
    (0x40, 2.0),
    (0x50, 8.0),                    # e = 10
    (0x78, 256.0),                  # e = 15, m = 0
    (0x7E, 448.0),                  # e = 15, m = 6: largest finite
    (0xB8, -1.0),
    (0xFE, -448.0),
]


def _finite_codes():
    return [c for c in range(256) if not math.isnan(oracle.e4m3_decode(c))]


def _brute_encode(x: float) -> int:
    """Nearest finite code to min(|x|, 448) with x's sign; on a tie the code
    whose last mantissa bit is 0."""
    if math.isnan(x):
        return 0x7F
    a = min(abs(x), 448.0)
    best = None
    for c in range(0x7F):                       # non-negative finite codes
        d = abs(oracle.e4m3_decode(c) - a)
        if best is None or d < best[0] or (d == best[0] and (c & 1) == 0):
            best = (d, c)
    return best[1] | (0x80 if math.copysign(1.0, x) < 0 else 0)


def test_hand_codes():
    for code, value in HAND_CODES:
        assert oracle.e4m3_decode(code) == value, hex(code)
    assert math.isnan(oracle.e4m3_decode(0x7F)) and math.isnan(oracle.e4m3_decode(0xFF))
    assert oracle.e4m3_decode(0x80) == 0.0 and math.copysign(1, oracle.e4m3_decode(0x80)) < 0
    assert len(_finite_codes()) == 254


def test_round_trip_every_finite_code():
    for c in _finite_codes():
        assert oracle.e4m3_encode(oracle.e4m3_decode(c)) == c, hex(c)
    codes = np.array(_finite_codes(), dtype=np.uint8)
    np.testing.assert_array_equal(oracle.e4m3_encode_array(oracle.e4m3_decode_array(codes)), codes)


def _probe_values():
    vals = []
    pos = sorted({oracle.e4m3_decode(c) for c in range(0x7F)})
    for lo, hi in zip(pos, pos[1:]):
        mid = (lo + hi) / 2.0                       # exact in float64
        vals += [lo, mid, hi, np.nextafter(mid, 0.0), np.nextafter(mid, 1e9)]
    vals += [448.0, 449.0, 463.99, 464.0, 464.01, 480.0, 1e6, 3e38,
             2.0 ** -10, 2.0 ** -10 + 2.0 ** -30, 2.0 ** -11, 1e-30, 0.0]
    rng = np.random.default_rng(17)
    vals += list(rng.normal(size=2000) * 10.0 ** rng.uniform(-4, 3, size=2000))
    vals = [float(np.float32(v)) for v in vals]     # inputs are float32 values
    return vals + [-v for v in vals] + [math.nan]


def test_encoder_matches_brute_force():
    vals = _probe_values()
    want = [_brute_encode(v) for v in vals]
    got = [oracle.e4m3_encode(v) for v in vals]
    assert got == want
    np.testing.assert_array_equal(oracle.e4m3_encode_array(np.array(vals)),
                                  np.array(want, dtype=np.uint8))


def test_ties_go_to_even_and_saturate():
    assert oracle.e4m3_encode(1.0625) == 0x38      # halfway 1.0 (m=0) / 1.125 (m=1)
    assert oracle.e4m3_encode(1.1875) == 0x3A      # halfway 1.125 (m=1) / 1.25 (m=2)
    assert oracle.e4m3_encode(2.0 ** -10) == 0x00  # half the smallest subnormal
    assert oracle.e4m3_encode(3 * 2.0 ** -10) == 0x02
    assert oracle.e4m3_encode(464.0) == 0x7E       # past 448 saturates
    assert oracle.e4m3_encode(-1e9) == 0xFE
    assert oracle.e4m3_encode(-2.0 ** -12) == 0x80  # negative, rounds to -0


def test_encoder_is_monotonic():
    x = np.sort(np.random.default_rng(3).normal(size=20000) * 50.0)
    v = oracle.e4m3_decode_array(oracle.e4m3_encode_array(x))
    assert np.all(np.diff(v) >= 0)


def test_quantize_divides_in_float32():
    one = np.array([0x3F80], dtype=np.uint16)      # bf16 1.0
    assert oracle.quantize(one, 0.5)[0] == 0x40    # 2.0
    # float32(1/3) = 0.333333343..., nearest E4M3 is 11/32 = 0.34375
    assert oracle.quantize(one, 3.0)[0] == 0x2B
    assert oracle.e4m3_decode(0x2B) == 0.34375
    x = np.random.default_rng(4).normal(size=5000).astype(np.float32)
    s = 0.0123
    want = np.array([_brute_encode(float(np.float32(v / np.float32(s)))) for v in x],
                    dtype=np.uint8)
    np.testing.assert_array_equal(oracle.quantize(x, s), want)


def test_fp8_decode_equals_pool_of_dequantised_values():
    rng = np.random.default_rng(9)
    N, Hkv, D, bs = 6, 2, 64, 16
    codes = rng.integers(0, 256, size=(N, 2, Hkv, bs, D), dtype=np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x38              # no NaN codes
    ks, vs = 0.037, 0.011
    deq = oracle.e4m3_decode_array(codes)
    deq[:, 0] *= ks
    deq[:, 1] *= vs
    q = rng.normal(size=(3, 8, D)).astype(np.float32)
    bt = np.array([[0, 1, 2], [3, 4, -1], [5, -1, -1]], dtype=np.int32)
    lens = [40, 17, 16]
    o8, l8 = oracle.decode(q, codes, bt, lens, 0.125, k_scale=ks, v_scale=vs)
    o64, l64 = oracle.decode(q, deq, bt, lens, 0.125)       # float64 pool of the values
    np.testing.assert_allclose(o8, o64, rtol=0, atol=1e-12)
    np.testing.assert_allclose(l8, l64, rtol=0, atol=1e-12)


def test_fp8_chunk_equals_pool_of_dequantised_values():
    """prefill_chunk over FP8 codes with cache scales equals the same chunk over
    a float64 pool holding code value x scale (the reading used for the rows
    a speculative step checks over an FP8 cache)."""
    rng = np.random.default_rng(10)
    N, Hkv, D, bs = 6, 2, 64, 16
    codes = rng.integers(0, 256, size=(N, 2, Hkv, bs, D), dtype=np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x38              # no NaN codes
    ks, vs = 0.029, 0.017
    deq = oracle.e4m3_decode_array(codes)
    deq[:, 0] *= ks
    deq[:, 1] *= vs
    lens, C = [40, 17, 16], 3
    q = rng.normal(size=(3 * C, 8, D)).astype(np.float32)
    qsl = np.arange(0, 3 * C + 1, C)
    bt = np.array([[0, 1, 2], [3, 4, -1], [5, -1, -1]], dtype=np.int32)
    o8, l8 = oracle.prefill_chunk(q, qsl, codes, bt, lens, 0.125, k_scale=ks, v_scale=vs)
    o64, l64 = oracle.prefill_chunk(q, qsl, deq, bt, lens, 0.125)
    np.testing.assert_allclose(o8, o64, rtol=0, atol=1e-12)
    np.testing.assert_allclose(l8, l64, rtol=0, atol=1e-12)
