"""FP8 (E4M3) KV-cache codec of the oracle -- TEST INFRASTRUCTURE.

The pages name an FP8 KV cache as a way to halve the cache's bytes but fix
no format or scale convention.  The reading used here (stated in full so a
reader can check it by eye):

* Format: the OCP 8-bit E4M3 encoding.  Bit 7 is the sign, bits 6..3 the
  exponent field e (bias 7), bits 2..0 the mantissa m.
    e == 0:          value = (-1)^s * m / 8 * 2^-6       (subnormals, zeros)
    0 < e, not NaN:  value = (-1)^s * (1 + m / 8) * 2^(e - 7)
    e == 15, m == 7: NaN (no infinities); the largest finite value is 448.
* Quantisation of a stored cache input x with a per-tensor scale s (one for
  keys, one for values): q = float32(x) / float32(s) computed in float32
  (IEEE division, round to nearest even), then |q| is saturated at 448 and
  rounded to the nearest E4M3 value, ties to the even mantissa; the sign is
  kept (a negative value that rounds to zero is stored as -0, code 0x80).
* Dequantisation: value(code) * s, exactly (float64).

Plain code, no tables shared with anything else; pinned in
tests/test_oracle_fp8.py against a brute-force nearest-code search and
hand-checked codes.
"""
import math

import numpy as np

E4M3_MAX = 448.0
_SUBNORMAL_QUANTUM = 2.0 ** -9    # m / 8 * 2^-6


def e4m3_decode(code: int) -> float:
    """Value of one E4M3 code (float, NaN for the two NaN codes)."""
    code = int(code) & 0xFF
    s = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return math.nan
    if e == 0:
        return s * m * _SUBNORMAL_QUANTUM
    return s * (1.0 + m / 8.0) * 2.0 ** (e - 7)


def _round_half_even(v: float) -> int:
    """Nearest integer to a non-negative float, ties to even (exact: the
    inputs here are float32 values divided by powers of two)."""
    f = math.floor(v)
    r = v - f
    if r > 0.5:
        return f + 1
    if r < 0.5:
        return f
    return f if f % 2 == 0 else f + 1


def e4m3_encode(x: float) -> int:
    """Code of float x: saturate |x| at 448, round to the nearest E4M3 value
    (ties to the even mantissa), keep the sign.  NaN gives 0x7F."""
    x = float(x)
    if math.isnan(x):
        return 0x7F
    sign = 0x80 if math.copysign(1.0, x) < 0 else 0
    a = min(abs(x), E4M3_MAX)
    if a == 0.0:
        return sign
    # spacing of E4M3 values around a: 2^-9 below 2^-6, else 2^(E - 3)
    E = math.frexp(a)[1] - 1              # a = f * 2^E with 1 <= f < 2
    quantum = _SUBNORMAL_QUANTUM if E < -6 else 2.0 ** (E - 3)
    r = _round_half_even(a / quantum) * quantum
    if r == 0.0:
        return sign
    # encode the exact value r (rounding may have carried into the next binade)
    E = math.frexp(r)[1] - 1
    if E < -6:
        return sign | int(r / _SUBNORMAL_QUANTUM)
    m = int(r / 2.0 ** (E - 3)) - 8
    assert 0 <= m <= 7 and 1 <= E + 7 <= 15
    return sign | ((E + 7) << 3) | m


def e4m3_decode_array(codes: np.ndarray) -> np.ndarray:
    """float64 values of an array of uint8 codes."""
    codes = np.asarray(codes, dtype=np.uint8)
    table = np.array([e4m3_decode(c) for c in range(256)], dtype=np.float64)
    return table[codes]


def e4m3_encode_array(q: np.ndarray) -> np.ndarray:
    """e4m3_encode applied to every element of a float array, written with
    numpy for test-sized pools: the same steps (saturate, spacing from the
    binade, round half to even, encode the rounded value)."""
    q = np.asarray(q, dtype=np.float64)
    nan = np.isnan(q)
    sign = np.where(np.signbit(q), 0x80, 0).astype(np.int64)
    a = np.minimum(np.abs(np.where(nan, 0.0, q)), E4M3_MAX)
    E = np.frexp(a)[1].astype(np.int64) - 1
    quantum = np.where(E < -6, _SUBNORMAL_QUANTUM, np.ldexp(1.0, np.maximum(E - 3, -1074)))
    r = np.rint(a / quantum) * quantum                    # numpy rint: ties to even
    E2 = np.frexp(r)[1].astype(np.int64) - 1
    sub = E2 < -6
    code_sub = np.rint(r / _SUBNORMAL_QUANTUM).astype(np.int64)
    mant = np.rint(r / np.ldexp(1.0, np.maximum(E2 - 3, -1074))).astype(np.int64) - 8
    code_norm = ((E2 + 7) << 3) | mant
    code = np.where(r == 0.0, 0, np.where(sub, code_sub, code_norm))
    code = np.where(nan, 0x7F, sign | code)
    return code.astype(np.uint8)


def quantize(x_stored: np.ndarray, scale: float) -> np.ndarray:
    """uint8 codes of stored cache inputs (bf16 bit patterns as uint16, or
    float32) under the per-tensor scale: float32 division, then the E4M3
    encoding (e4m3_encode_array)."""
    x = np.asarray(x_stored)
    if x.dtype == np.uint16:
        x32 = (x.astype(np.uint32) * np.uint32(65536)).view(np.float32)
    elif x.dtype == np.float32:
        x32 = x
    else:
        raise TypeError(f"unsupported input element type {x.dtype}")
    q = (x32 / np.float32(scale)).astype(np.float32)   # IEEE float32 division
    return e4m3_encode_array(q)
