"""Number formats used on the path, written from their definitions (oracle; test-only).

* bf16: the upper 16 bits of an IEEE binary32; rounding to nearest, ties to even.
* fp16: IEEE binary16 (numpy's float16 cast, round-to-nearest-even, is the library step).
* e4m3 ("fp8 E4M3FN" of the OCP 8-bit floating point spec): 1 sign, 4 exponent bits with
  bias 7, 3 mantissa bits; no infinities; S.1111.111 is NaN, so the largest finite
  magnitude is 1.75 * 2^8 = 448; exponent field 0 holds subnormals m/8 * 2^-6.
  Encoding rounds to nearest, ties to even, and saturates to +-448 (inputs here are
  clamped to +-448 first, as the fp8 quantizer does).
Pins: tests/test_oracle_formats.py (against torch's casts, exhaustively).
"""
import numpy as np


def bf16_encode(x) -> np.ndarray:
    """float32 values -> bf16 bit patterns (uint16), round to nearest even. Finite inputs."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = (u + 0x7FFF + lsb) >> 16
    return r.astype(np.uint16)


def bf16_decode(bits) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64 (exact)."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    with np.errstate(invalid="ignore"):          # NaN patterns widen to NaN
        return u.view(np.float32).astype(np.float64)


def fp16_round(x) -> np.ndarray:
    """Round to IEEE binary16 (nearest even) and return as float64 (exact)."""
    return np.asarray(x, dtype=np.float64).astype(np.float16).astype(np.float64)


E4M3_MAX = 448.0


def e4m3_decode(codes) -> np.ndarray:
    """e4m3 codes (uint8) -> float64 (exact). NaN codes decode to nan."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    val = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    val = np.where((c & 0x7F) == 0x7F, np.nan, val)
    return sign * val


def e4m3_encode(x) -> np.ndarray:
    """Finite values -> e4m3 codes (uint8): round to nearest even, saturate at 448."""
    x = np.asarray(x, dtype=np.float64)
    sign = (np.signbit(x)).astype(np.int64) << 7
    a = np.minimum(np.abs(x), E4M3_MAX)
    out = np.zeros(a.shape, dtype=np.int64)
    sub = a < 2.0 ** -6
    # subnormal range: multiples of 2^-9; m == 8 rolls into the smallest normal (code 0x08)
    out[sub] = np.rint(a[sub] / 2.0 ** -9).astype(np.int64)
    nrm = ~sub
    f, ex = np.frexp(a[nrm])             # a = f * 2^ex, f in [0.5, 1)
    e = ex.astype(np.int64) - 1          # a = (2f) * 2^e, 2f in [1, 2)
    m = np.rint((2.0 * f - 1.0) * 8.0).astype(np.int64)
    carry = m == 8
    e = e + carry
    m = np.where(carry, 0, m)
    out[nrm] = ((e + 7) << 3) | m
    return (out | sign).astype(np.uint8)
