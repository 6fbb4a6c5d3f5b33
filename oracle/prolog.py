"""Indexer prolog (oracle; test-only): RoPE -> Hadamard -> per-token-head dynamic quant.

[PRO] "Indexer Prolog", formulas: the indexer query and the indexer cache key are each
quantized per token-head after a Hadamard transform that follows RoPE; the query is A8,
the cache C8, and dequant factors are stored in FP16.  The Hadamard is applied as a
right-multiplication by a Hadamard matrix.  The upstream projections (q . w_qb with its
W8A8 dequant, x . w_k followed by LayerNorm) are outside this step: the inputs here are
the projected activations.

[AQ] "Activation Quantization", steps 1-3: convert to fp32, take |x|, reduce to the row
maximum, scale = max / 127 (optionally rounded to a power of two), y = round(clamp(x /
scale, -127, 127)).  The fp8 variant uses 448 (the e4m3 maximum) in place of 127.

Readings (where the pages leave a step open):
  * RoPE acts on `rope_dim` dims starting at `rope_offset`; pairs are (i, i + rope_dim/2)
    unless `interleaved` (then (2i, 2i+1)); cos/sin are caller inputs.
  * The Hadamard matrix is Sylvester's, H[i, j] = (-1)^popcount(i & j) / sqrt(D)
    (orthonormal, natural order).
  * RoPE and Hadamard are computed in float64 and the result is rounded once to fp32,
    where the quantizer (fixed at fp32 by [AQ]) takes over.
  * Granularity is one scale per (token, head) over its D dims ("Per-Token-Head").
  * round() is round-half-to-even; amax == 0 gives scale 0 and all-zero codes.
  * The fp32 scale is used for the codes; the stored scale is that value rounded to the
    scale dtype (fp16 by [PRO], or fp32).
Pins: tests/test_oracle_prolog.py (each step alone) and tests/test_oracle_compose.py (the
chain's order through closed-form unit-vector cases; the per-token rotary broadcast over
the query heads).
"""
import numpy as np

from .formats import e4m3_encode, fp16_round


def hadamard(n: int) -> np.ndarray:
    """Orthonormal Sylvester-Hadamard matrix of order n (power of two), float64."""
    assert n > 0 and (n & (n - 1)) == 0
    i = np.arange(n)
    bits = np.bitwise_and(i[:, None], i[None, :])
    pop = np.zeros_like(bits)
    while np.any(bits):
        pop += bits & 1
        bits >>= 1
    return np.where(pop % 2 == 0, 1.0, -1.0) / np.sqrt(float(n))


def apply_rope(x: np.ndarray, cos: np.ndarray, sin: np.ndarray, rope_dim: int,
               rope_offset: int, interleaved: bool) -> np.ndarray:
    """Rotate pairs of x[..., rope_offset : rope_offset + rope_dim] (float64).

    x: [R, D] float64; cos, sin: [R, rope_dim/2].  Pair i (x1, x2) becomes
    (x1 cos_i - x2 sin_i, x2 cos_i + x1 sin_i).
    """
    y = np.array(x, dtype=np.float64, copy=True)
    half = rope_dim // 2
    idx = np.arange(half)
    if interleaved:
        i1, i2 = rope_offset + 2 * idx, rope_offset + 2 * idx + 1
    else:
        i1, i2 = rope_offset + idx, rope_offset + half + idx
    c = np.asarray(cos, dtype=np.float64)
    s = np.asarray(sin, dtype=np.float64)
    x1, x2 = x[:, i1], x[:, i2]
    y[:, i1] = x1 * c - x2 * s
    y[:, i2] = x2 * c + x1 * s
    return y


def quantize_rows(x32: np.ndarray, code: str, scale_dt: str, round_scale: bool = False):
    """Per-row symmetric dynamic quantization in fp32 ([AQ] steps 1-3).

    x32: [R, D] float32.  Returns (codes, scale_stored_f64, scale_f32):
      codes int8 values (as int8) for code == "i8", or e4m3 codes (uint8) for "e4m3";
      scale_stored: the fp32 scale rounded to scale_dt ("f16" | "f32"), as float64.
    """
    x32 = np.asarray(x32, dtype=np.float32)
    qmax = np.float32(127.0) if code == "i8" else np.float32(448.0)
    amax = np.max(np.abs(x32), axis=-1)                               # exact in fp32
    s = (amax / qmax).astype(np.float32)                              # fp32 division
    if round_scale:
        # power of two not below s: keeps |x / s| <= qmax
        f, e = np.frexp(s.astype(np.float64))            # s = f * 2^e, f in [0.5, 1)
        up = np.where(f == 0.5, np.ldexp(1.0, e - 1), np.ldexp(1.0, e))
        s = np.where(s > 0, up, 0.0).astype(np.float32)
    safe = np.where(s > 0, s, np.float32(1.0)).astype(np.float32)
    y = (x32 / safe[:, None]).astype(np.float32)                      # fp32 division
    y = np.clip(y, -qmax, qmax)
    y = np.where((s > 0)[:, None], y, np.float32(0.0))
    if code == "i8":
        codes = np.rint(y).astype(np.int8)
    else:
        codes = e4m3_encode(y)
    stored = fp16_round(s) if scale_dt == "f16" else s.astype(np.float64)
    return codes, stored, s


def prolog_rows(x_in: np.ndarray, cos, sin, rope_dim: int, rope_offset: int,
                interleaved: bool, use_hadamard: bool, code: str, scale_dt: str,
                round_scale: bool = False):
    """One quantized row per input row: RoPE (if rope_dim) -> Hadamard (if asked) -> fp32 -> quant.

    x_in: [R, D] raw activations (float32 values; bf16 inputs already widened exactly).
    """
    x = np.asarray(x_in, dtype=np.float64)
    if rope_dim:
        x = apply_rope(x, cos, sin, rope_dim, rope_offset, interleaved)
    if use_hadamard:
        x = x @ hadamard(x.shape[-1])
    x32 = x.astype(np.float32)                                        # one rounding to fp32
    return quantize_rows(x32, code, scale_dt, round_scale)


def indexer_prolog(q_in, k_in, q_cos, q_sin, k_cos, k_sin, rope_dim, rope_offset,
                   interleaved, use_hadamard, code, scale_dt, round_scale=False):
    """[PRO] both streams: q_in [T, H, D] -> q codes [T, H, D], q scales [T, H];
    k_in [R, D] -> k codes [R, D], k scales [R].  Either input may be None."""
    out = {}
    if q_in is not None:
        T, H, D = q_in.shape
        qc = np.repeat(q_cos, H, axis=0) if rope_dim else None
        qs = np.repeat(q_sin, H, axis=0) if rope_dim else None
        c, s, _ = prolog_rows(q_in.reshape(T * H, D), qc, qs, rope_dim, rope_offset,
                              interleaved, use_hadamard, code, scale_dt, round_scale)
        out["q_codes"], out["q_scale"] = c.reshape(T, H, D), s.reshape(T, H)
    if k_in is not None:
        c, s, _ = prolog_rows(k_in, k_cos, k_sin, rope_dim, rope_offset, interleaved,
                              use_hadamard, code, scale_dt, round_scale)
        out["k_codes"], out["k_scale"] = c, s
    return out
