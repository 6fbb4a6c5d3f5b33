"""Pins for oracle/formats.py against library casts (torch, numpy), exhaustively where cheap."""
import numpy as np
import torch

from oracle.formats import bf16_decode, bf16_encode, e4m3_decode, e4m3_encode, fp16_round


def test_bf16_encode_matches_torch_random_bits(rng):
    bits = rng.integers(0, 2**32, size=1 << 20, dtype=np.uint64).astype(np.uint32)
    x = bits.view(np.float32)
    x = x[np.isfinite(x) & (np.abs(x) < 3.0e38)]
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(bf16_encode(x), ref)


def test_bf16_encode_ties_to_even():
    # 1 + 2^-8 is halfway between bf16 neighbours 1 and 1 + 2^-7 -> even (1.0)
    x = np.array([1 + 2**-8, 1 + 3 * 2**-8, -(1 + 2**-8), 0.0, -0.0], dtype=np.float32)
    got = bf16_decode(bf16_encode(x))
    assert got.tolist() == [1.0, 1 + 2**-6, -1.0, 0.0, -0.0]


def test_bf16_decode_exact_roundtrip(rng):
    b = rng.integers(0, 2**16, size=1 << 16, dtype=np.uint64).astype(np.uint16)
    v = bf16_decode(b)
    ok = np.isfinite(v)
    assert np.array_equal(bf16_encode(v[ok].astype(np.float32)), b[ok])


def test_e4m3_decode_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = e4m3_decode(codes)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok])
    assert np.nanmax(got) == 448.0 and e4m3_decode(np.array([1], np.uint8))[0] == 2.0**-9


def _torch_e4m3(x32):
    return torch.from_numpy(x32).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_e4m3_encode_all_bf16_in_range_match_torch():
    b = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    x = (b.astype(np.uint32) << 16).view(np.float32)
    x = x[np.isfinite(x) & (np.abs(x) <= 448.0)]
    assert np.array_equal(e4m3_encode(x), _torch_e4m3(x))


def test_e4m3_encode_random_f32_and_exact_midpoints_match_torch(rng):
    x = (rng.uniform(-448, 448, size=1 << 20)).astype(np.float32)
    small = (rng.standard_normal(1 << 18) * 2.0**-7).astype(np.float32)   # subnormal range
    vals = e4m3_decode(np.arange(0, 0x7E, dtype=np.uint8))                  # 0 .. 416
    mids = ((vals[:-1] + vals[1:]) / 2).astype(np.float32)                  # exact ties
    allx = np.concatenate([x, small, mids, -mids])
    assert np.array_equal(e4m3_encode(allx), _torch_e4m3(allx))


def test_e4m3_encode_saturates():
    assert e4m3_encode(np.array([448.0, 1e9, -1e9]))[0] == 0x7E
    assert e4m3_encode(np.array([1e9]))[0] == 0x7E and e4m3_encode(np.array([-1e9]))[0] == 0xFE


def test_fp16_round_definition():
    got = fp16_round(np.array([1 + 2**-11, 1 + 3 * 2**-11, 65504.0, 2.0**-24, 1 / 3]))
    assert got[0] == 1.0 and got[1] == 1 + 2**-9 and got[2] == 65504.0 and got[3] == 2.0**-24
    assert abs(got[4] - 1 / 3) <= 2**-12 / 3
