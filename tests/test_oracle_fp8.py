"""Pins of the oracle's FP8 latent cache ([AUDIT] §6.1 lists an FP8 KV cache in
FlashMLA's support matrix; the format and per-token scale are the reading the
oracle documents) against what the format definition, a library conversion and
brute force fix.

* E4M3 decoding of all 256 codes and encoding of random values, of every
  rounding midpoint and of its neighbours, against torch's float8_e4m3fn
  conversion on the CPU (a library routine);
* encoding against a pure-Python nearest-value search over the 256 codes;
* per-token quantization: the scale is the smallest power of two that
  brings the row's largest element within +-448 (so it lands in (224, 448]
  before rounding),
  with exponent at least -124, checked at the boundaries and against a
  search over exponents; rows made of codes times a power of two come back
  unchanged, and the dequantized row stays within half a grid step of the
  input;
* the FP8 decode equals the naive (expanding) path run on the dequantized rows
  with their rope part rotated back (fp64, 1e-10);
* planted mistakes in the quantizer (round half away from zero, no scale,
  a scale one power of two too large, rope left out) fail these pins.

Tags: [AUDIT] llm-atlas "DeepSeek MLA 吸收式缓存：真实权重执行与 FlashMLA 架构边界".
"""

import math

import numpy as np
import pytest
import torch

from oracle import mla


def torch_encode(x):
    return torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def all_finite_values():
    codes = np.arange(256, dtype=np.uint8)
    v = mla.e4m3_decode(codes)
    return np.unique(v[np.isfinite(v) & (v >= 0)])


# ---------------------------------------------------------------------------- pins as functions


def check_decode_table():
    codes = np.arange(256, dtype=np.uint8)
    ours = mla.e4m3_decode(codes)
    lib = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(ours), np.isnan(lib))
    assert np.array_equal(ours[~np.isnan(ours)], lib[~np.isnan(lib)])
    assert mla.e4m3_decode(np.uint8(0x7E)) == 448.0 and mla.e4m3_decode(np.uint8(0x01)) == 2.0 ** -9


def check_encode_random():
    rng = np.random.default_rng(1)
    x = np.concatenate([
        rng.standard_normal(200_000) * 30.0,
        rng.standard_normal(50_000) * 2.0 ** -7,      # subnormal range
        rng.uniform(-448, 448, 50_000),
    ]).astype(np.float32)
    x = np.clip(x, -448.0, 448.0).astype(np.float32)
    assert np.array_equal(mla.e4m3_encode(x), torch_encode(x))


def check_encode_midpoints():
    v = all_finite_values()
    mid = ((v[:-1] + v[1:]) / 2).astype(np.float32)     # exact in float32
    near = np.concatenate([mid, np.nextafter(mid, np.float32(0)), np.nextafter(mid, np.float32(1e9))])
    x = np.concatenate([near, -near, v.astype(np.float32), -v.astype(np.float32)]).astype(np.float32)
    assert np.array_equal(mla.e4m3_encode(x), torch_encode(x))


def check_encode_brute_force():
    """Nearest code by exhaustive search; a tie goes to the even mantissa
    (the code with bit 0 clear)."""
    codes = np.arange(0, 0x7F, dtype=np.uint8)          # non-negative finite codes
    vals = mla.e4m3_decode(codes)
    rng = np.random.default_rng(2)
    xs = np.concatenate([rng.standard_normal(2000) * 40, rng.standard_normal(500) * 0.01])
    xs = np.concatenate([xs, (vals[:-1] + vals[1:]) / 2]).astype(np.float32)
    xs = np.clip(xs, -448, 448).astype(np.float32)
    got = mla.e4m3_encode(xs)
    for x, g in zip(xs.tolist(), got.tolist()):
        a = abs(x)
        d = np.abs(vals - a)
        best = np.flatnonzero(d == d.min())
        c = int(best[0]) if len(best) == 1 else int([b for b in best if b % 2 == 0][0])
        if x < 0 or (x == 0 and math.copysign(1, x) < 0):
            c |= 0x80
        assert g == c, (x, g, c)


def check_saturation():
    x = np.array([448.0, 449.0, 463.9, -455.0], dtype=np.float32)
    assert mla.e4m3_encode(x).tolist() == [0x7E, 0x7E, 0x7E, 0xFE]


def check_row_quantization():
    rng = np.random.default_rng(3)
    rows = (rng.standard_normal((300, 576)) * rng.uniform(1e-3, 1e3, (300, 1))).astype(np.float32)
    rows[7] = 0.0
    codes, scale = mla.quantize_rows_fp8(rows)
    deq = mla.dequantize_rows_fp8(codes, scale)
    mags = np.abs(mla.e4m3_decode(codes))
    nz = np.any(rows != 0, axis=1)
    amax = np.abs(rows).max(axis=1).astype(np.float64)
    s64 = scale.astype(np.float64)
    # a power of two, the smallest with amax / scale <= 448
    assert np.all(np.frexp(s64)[0] == 0.5)
    assert np.all(amax[nz] / s64[nz] <= 448.0) and np.all(amax[nz] / (s64[nz] / 2) > 448.0)
    # so the largest element of each nonzero row lands in (224, 448] before
    # rounding, on a code in [224, 448] after it (the grid step there is 16)
    top = mags[nz].max(axis=1)
    assert np.all((top >= 224.0) & (top <= 448.0))
    assert scale[7] == 1.0 and np.all(codes[7] == 0)
    # half a grid step: 2^-4 relative in the normal range, 2^-10 scale below it
    r64 = rows.astype(np.float64)
    bound = np.maximum(np.abs(r64) * 2.0 ** -4, scale[:, None].astype(np.float64) * 2.0 ** -10)
    assert np.all(np.abs(deq - r64) <= bound * (1 + 1e-6))


def check_token_scale():
    """Boundaries of the power-of-two scale, and a search over exponents."""
    f32 = np.float32
    cases = {448.0: 1.0, 224.0: 0.5, 0.875: 2.0 ** -9, 896.0: 2.0, 1.0: 2.0 ** -8, 2.0 ** 100 * 448: 2.0 ** 100}
    for a, want in cases.items():
        assert mla.fp8_token_scale(f32(a)) == f32(want), a
    assert mla.fp8_token_scale(np.nextafter(f32(448), f32(1e9))) == f32(2.0)
    assert mla.fp8_token_scale(np.nextafter(f32(224), f32(1e9))) == f32(1.0)
    assert mla.fp8_token_scale(f32(0)) == f32(1.0)
    assert mla.fp8_token_scale(f32(1e-40)) == f32(2.0 ** -124)   # float32 subnormal amax: the floor
    rng = np.random.default_rng(7)
    a = (np.abs(rng.standard_normal(5000)) * np.exp2(rng.uniform(-100, 100, 5000))).astype(np.float32)
    got = mla.fp8_token_scale(a).astype(np.float64)
    for x, g in zip(a.astype(np.float64).tolist(), got.tolist()):
        k = next(k for k in range(-124, 129) if x / 2.0 ** k <= 448.0)
        assert g == 2.0 ** k, (x, g, k)


def check_round_trip_exact():
    """Rows that are E4M3 values times 2^k with a +-448 entry come back unchanged."""
    rng = np.random.default_rng(4)
    finite = np.flatnonzero(np.isfinite(mla.e4m3_decode(np.arange(256, dtype=np.uint8))))
    codes = rng.choice(finite, (20, 576)).astype(np.uint8)
    codes[:, 5] = 0x7E
    k = rng.integers(-12, 12, 20)
    rows = (mla.e4m3_decode(codes) * np.ldexp(1.0, k)[:, None]).astype(np.float32)
    c2, s2 = mla.quantize_rows_fp8(rows)
    assert np.array_equal(s2, np.ldexp(1.0, k).astype(np.float32))
    assert np.array_equal(mla.e4m3_decode(c2), mla.e4m3_decode(codes))


def check_cache_rows_fp8():
    rng = np.random.default_rng(5)
    L = 40
    c_kv = rng.standard_normal((L, 512)).astype(np.float32).astype(np.float64)
    k_pe = rng.standard_normal((L, 64))
    pos = np.arange(1000, 1000 + L)
    codes, scale = mla.cache_rows_fp8(c_kv, k_pe, pos)
    ref = np.concatenate([c_kv, mla.rope(k_pe, pos)], axis=-1)   # rope pinned in test_oracle_math
    deq = mla.dequantize_rows_fp8(codes, scale)
    bound = np.maximum(np.abs(ref) * 2.0 ** -4, scale[:, None] * 2.0 ** -10) * (1 + 1e-6) + 1e-7 * np.abs(ref)
    assert np.all(np.abs(deq - ref) <= bound)


def check_decode_fp8_vs_naive():
    rng = np.random.default_rng(6)
    H, Lq, L = 4, 3, 70
    c_kv = rng.standard_normal((L, 512))
    k_pe = rng.standard_normal((L, 64))
    q_nope = rng.standard_normal((Lq, H, 128))
    q_pe = rng.standard_normal((Lq, H, 64))
    w_uk = rng.standard_normal((H, 128, 512)) / math.sqrt(512)
    w_uv = rng.standard_normal((H, 128, 512)) / math.sqrt(512)
    codes, scale = mla.cache_rows_fp8(c_kv, k_pe, np.arange(L))
    got = mla.absorbed_decode_fp8(q_nope, q_pe, codes, scale, w_uk, w_uv)
    rows = mla.e4m3_decode(codes) * scale.astype(np.float64)[:, None]
    # rotate the stored rope keys back to position 0: R(t)^-1 = R(-t)
    k_pe_back = mla.rope(rows[:, 512:], -np.arange(L))
    ref = mla.naive_decode(q_nope, q_pe, rows[:, :512], k_pe_back, w_uk, w_uv)
    tol = 1e-10 * max(1.0, np.abs(ref["o"]).max())
    assert np.abs(got["o"] - ref["o"]).max() <= tol
    assert np.abs(got["lse"] - ref["lse"]).max() <= 1e-10 * max(1.0, np.abs(ref["lse"]).max())


# ---------------------------------------------------------------------------- the pins


def test_e4m3_decode_table():
    check_decode_table()


def test_e4m3_encode_random_vs_torch():
    check_encode_random()


def test_e4m3_encode_midpoints_vs_torch():
    check_encode_midpoints()


def test_e4m3_encode_brute_force():
    check_encode_brute_force()


def test_e4m3_saturation():
    check_saturation()


def test_row_quantization_bounds():
    check_row_quantization()


def test_token_scale_power_of_two():
    check_token_scale()


def test_row_quantization_round_trip():
    check_round_trip_exact()


def test_cache_rows_fp8_within_grid():
    check_cache_rows_fp8()


def test_fp8_decode_equals_naive_on_dequantized_rows():
    check_decode_fp8_vs_naive()


def test_fp8_cache_accounting():
    """Bytes per token: 576 one-byte codes and a 4-byte scale against 576
    bf16 values; 64-token blocks of 36,864 code bytes."""
    assert mla.mla_cache_elems_per_token() == 576
    assert mla.mla_bytes_per_token(elt=1) + 4 == 580
    assert mla.mla_bytes_per_token(elt=2) == 1152
    assert mla.paged_allocated_bytes(26, mla.mla_bytes_per_token(elt=1)) == 36864


# ---------------------------------------------------------------------------- planted mistakes


def test_planted_round_half_away(monkeypatch):
    real = np.rint
    monkeypatch.setattr(mla.np, "rint", lambda x: np.sign(x) * np.floor(np.abs(x) + 0.5))
    with pytest.raises(AssertionError):
        check_encode_midpoints()
    monkeypatch.setattr(mla.np, "rint", real)


def test_planted_missing_scale(monkeypatch):
    monkeypatch.setattr(mla, "FP8_MAX", 1.0)
    with pytest.raises(AssertionError):
        check_row_quantization()


def test_planted_scale_too_large(monkeypatch):
    real = mla.fp8_token_scale
    monkeypatch.setattr(mla, "fp8_token_scale", lambda a: (real(a) * 2).astype(np.float32))
    with pytest.raises(AssertionError):
        check_row_quantization()
    with pytest.raises(AssertionError):
        check_token_scale()


def test_planted_rope_left_out(monkeypatch):
    real = mla.cache_rows
    monkeypatch.setattr(mla, "cache_rows",
                        lambda c, k, p, base=mla.ROPE_BASE: np.concatenate([np.asarray(c, np.float64),
                                                                           np.asarray(k, np.float64)], -1))
    with pytest.raises(AssertionError):
        check_cache_rows_fp8()
    monkeypatch.setattr(mla, "cache_rows", real)
