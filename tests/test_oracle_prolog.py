"""Pins for oracle/prolog.py: Hadamard, RoPE, per-token-head quantization."""
import numpy as np
import scipy.linalg

from oracle.formats import e4m3_decode
from oracle.prolog import apply_rope, hadamard, prolog_rows, quantize_rows


def test_hadamard_is_sylvester_orthonormal():
    for n in (2, 8, 64, 128):
        H = hadamard(n)
        assert np.allclose(H, scipy.linalg.hadamard(n) / np.sqrt(n), atol=0, rtol=0)
        assert np.allclose(H @ H.T, np.eye(n), atol=1e-15)
        assert np.array_equal(H, H.T)
        assert np.allclose(H @ H, np.eye(n), atol=1e-15)


def test_hadamard_preserves_dot_products(rng):
    x, y = rng.standard_normal((2, 5, 128))
    H = hadamard(128)
    assert np.allclose(np.sum((x @ H) * (y @ H), -1), np.sum(x * y, -1), rtol=1e-13)


def _tables(pos, rd, base=10000.0):
    inv = base ** (-np.arange(rd // 2) * 2.0 / rd)
    a = np.asarray(pos, dtype=np.float64)[:, None] * inv[None, :]
    return np.cos(a), np.sin(a)


def test_rope_identity_at_position_zero(rng):
    x = rng.standard_normal((3, 128))
    c, s = _tables([0, 0, 0], 64)
    for inter in (False, True):
        assert np.array_equal(apply_rope(x, c, s, 64, 64, inter), x)


def test_rope_matches_complex_rotation(rng):
    x = rng.standard_normal((4, 128))
    c, s = _tables([1, 7, 300, 65535], 64)
    y = apply_rope(x, c, s, 64, 64, False)
    z = (x[:, 64:96] + 1j * x[:, 96:128]) * (c + 1j * s)
    assert np.allclose(y[:, 64:96], z.real, atol=1e-12) and np.allclose(y[:, 96:128], z.imag, atol=1e-12)
    assert np.array_equal(y[:, :64], x[:, :64])          # nope dims untouched
    yi = apply_rope(x, c, s, 64, 64, True)
    zi = (x[:, 64:128:2] + 1j * x[:, 65:128:2]) * (c + 1j * s)
    assert np.allclose(yi[:, 64:128:2], zi.real, atol=1e-12)
    assert np.allclose(yi[:, 65:128:2], zi.imag, atol=1e-12)


def test_rope_relative_position(rng):
    x, y = rng.standard_normal((2, 1, 128))
    def dot(p1, p2):
        c1, s1 = _tables([p1], 64)
        c2, s2 = _tables([p2], 64)
        return float(np.sum(apply_rope(x, c1, s1, 64, 64, False) * apply_rope(y, c2, s2, 64, 64, False)))
    assert abs(dot(10, 3) - dot(1007, 1000)) < 1e-10
    assert abs(dot(5, 5) - float(np.sum(x * y))) < 1e-10


def test_int8_quant_hand_case():
    # amax 127 gives scale exactly 1.0: codes are round-half-even of the clamped values
    x = np.array([[127.0, 2.5, -3.5, 0.49, -126.6, 3.5]], dtype=np.float32)
    codes, stored, s = quantize_rows(x, "i8", "f16")
    assert codes.tolist() == [[127, 2, -4, 0, -127, 4]]
    assert stored.tolist() == [1.0] and s.tolist() == [1.0]


def test_int8_quant_invariants(rng):
    x = (rng.standard_normal((64, 128)) * rng.uniform(0.01, 100, (64, 1))).astype(np.float32)
    codes, stored, s = quantize_rows(x, "i8", "f32")
    assert codes.dtype == np.int8 and np.abs(codes.astype(int)).max() <= 127
    am = np.argmax(np.abs(x), axis=1)
    assert np.all(np.abs(codes[np.arange(64), am].astype(int)) == 127)
    err = np.abs(x.astype(np.float64) - codes * s[:, None].astype(np.float64))
    assert np.all(err <= s[:, None] * (0.5 + 1e-6))
    c2, _, s2 = quantize_rows((x * np.float32(8.0)).astype(np.float32), "i8", "f32")
    assert np.array_equal(c2, codes) and np.array_equal(s2, s * np.float32(8.0))


def test_quant_zero_row():
    codes, stored, s = quantize_rows(np.zeros((2, 8), np.float32), "i8", "f16")
    assert not codes.any() and not stored.any()
    codes, stored, s = quantize_rows(np.zeros((1, 8), np.float32), "e4m3", "f16")
    assert not codes.any()


def test_fp16_scale_storage_and_round_scale(rng):
    x = rng.standard_normal((32, 128)).astype(np.float32)
    _, stored, s = quantize_rows(x, "i8", "f16")
    assert np.array_equal(stored, s.astype(np.float16).astype(np.float64))
    codes, _, sp = quantize_rows(x, "i8", "f32", round_scale=True)
    m, e = np.frexp(sp)
    assert np.all(m == 0.5) and np.all(sp >= s) and np.all(sp < 2 * s)
    assert np.abs(codes.astype(int)).max() <= 127


def test_e4m3_quant_invariants(rng):
    x = (rng.standard_normal((64, 128)) * 3).astype(np.float32)
    codes, stored, s = quantize_rows(x, "e4m3", "f16")
    v = e4m3_decode(codes)
    am = np.argmax(np.abs(x), axis=1)
    assert np.all(np.abs(v[np.arange(64), am]) == 448.0)
    y = x.astype(np.float64) / s[:, None].astype(np.float64)
    nrm = np.abs(y) >= 2.0**-6
    assert np.all(np.abs(v - y)[nrm] <= np.abs(y)[nrm] * 2.0**-4 * (1 + 1e-6))
    assert np.all(np.abs(v - y)[~nrm] <= 2.0**-10 * (1 + 1e-6))


def test_prolog_rows_hadamard_codes_are_scale_free(rng):
    # codes depend on x only through x / amax: scaling the input by 2 leaves them unchanged
    x = rng.standard_normal((16, 128)).astype(np.float32)
    c, sn = _tables(np.arange(16), 64)
    a, _, s1 = prolog_rows(x, c, sn, 64, 64, False, True, "i8", "f16")
    b, _, s2 = prolog_rows(2 * x, c, sn, 64, 64, False, True, "i8", "f16")
    assert np.array_equal(a, b) and np.allclose(s2, 2 * s1, rtol=1e-6)
