"""Pins for the E4M3 codec of the oracle (oracle/fp8.py) and its FP8 decode path (CPU only).

* the format's defining values (tests/golden/e4m3_values.json, from the OCP
  8-bit floating-point specification) and its rounding cases;
* all 256 codes against torch's float8_e4m3fn conversion (a library routine);
* quantisation of every finite bf16 value within ±448 and of random fp32
  values at a non-power-of-two scale against torch's float8_e4m3fn cast;
* brute force: the chosen code is the nearest finite value, ties to the even
  mantissa;
* round trip of every finite code; monotone value table;
* the FP8 decode path equals the bf16 path exactly when the values are
  E4M3-exact and the scale is 1;
* planted mistakes in the codec table must fail the pins.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle.fp8 as F8
import oracle.attention as OA

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "e4m3_values.json")))
torch = pytest.importorskip("torch")


def _same(a, b):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    return np.array_equal(np.isnan(a), np.isnan(b)) and np.array_equal(
        np.where(np.isnan(a), 0, a), np.where(np.isnan(b), 0, b)) and np.array_equal(
        np.signbit(np.where(np.isnan(a), 0, a)), np.signbit(np.where(np.isnan(b), 0, b)))


@pytest.mark.parametrize("code,value", GOLD["values"])
def test_defining_values(code, value):
    assert _same(F8.e4m3_value(int(code, 16)), float(value))
    assert _same(F8.decode_e4m3(np.array([int(code, 16)], np.uint8))[0], float(value))


@pytest.mark.parametrize("x,code,why", GOLD["rounding"])
def test_rounding_cases(x, code, why):
    assert int(F8.quantize_e4m3(np.array([float(x)], np.float32), 1.0)[0]) == int(code, 16), why


def _torch_codes(q32):
    t = torch.from_numpy(np.ascontiguousarray(q32, dtype=np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float32).numpy()
    assert _same(F8.decode_e4m3(codes), ref)


def _finite_bf16_in_range():
    u = np.arange(65536, dtype=np.uint32)
    f = (u << 16).view(np.float32)
    keep = np.isfinite(f) & (np.abs(f) <= 448.0) & ((np.abs(f) >= np.float32(1.2e-38)) | (f == 0))
    return f[keep]


def test_quantize_every_bf16_matches_torch():
    x = _finite_bf16_in_range()
    assert len(x) > 30000
    assert np.array_equal(F8.quantize_e4m3(x, 1.0), _torch_codes(x))


def test_quantize_nan_keeps_nan_and_sign():
    """Every bf16 NaN pattern (both signs, any payload) gives the NaN code
    with its sign, as torch's float8_e4m3fn conversion does; clamping must
    not turn a NaN into ±448."""
    bits = np.arange(1 << 16, dtype=np.uint32)
    x = (bits << np.uint32(16)).view(np.float32)
    nan = x[np.isnan(x)]
    assert len(nan) == 2 * 127
    codes = F8.quantize_e4m3(nan, 1.0)
    assert np.array_equal(codes, _torch_codes(nan))
    assert set(codes.tolist()) == {0x7F, 0xFF}
    assert np.array_equal(codes == 0xFF, np.signbit(nan))
    assert np.array_equal(F8.quantize_e4m3(nan, 0.0137), codes)


@pytest.mark.parametrize("scale", [0.0137, 0.0129, 3.0, 2.0 ** -7])
def test_quantize_scaled_matches_torch(scale):
    rng = np.random.default_rng(7)
    x = (rng.standard_normal(200000) * rng.choice([0.01, 1.0, 5.0], 200000)).astype(np.float32)
    q = np.clip(x / np.float32(scale), -448, 448).astype(np.float32)
    assert np.array_equal(F8.quantize_e4m3(x, scale), _torch_codes(q))


def test_quantize_is_nearest_with_ties_to_even_brute_force():
    rng = np.random.default_rng(3)
    vals = F8.e4m3_table()
    finite = [c for c in range(256) if not math.isnan(vals[c])]
    xs = list(rng.standard_normal(1500).astype(np.float32) * 40)
    # exact midpoints between neighbouring positive values
    pos = sorted({vals[c] for c in finite if vals[c] > 0})
    xs += [np.float32((a + b) / 2) for a, b in zip(pos[:-1], pos[1:]) if np.float32((a + b) / 2) == (a + b) / 2]
    for x in xs:
        x = np.float32(x)
        got = int(F8.quantize_e4m3(np.array([x]), 1.0)[0])
        xv = float(np.clip(x, -448, 448))
        sign = 0x80 if np.signbit(xv) else 0
        same_sign = [c for c in finite if (c & 0x80) == sign]     # the sign is kept
        dist = {c: abs(abs(xv) - abs(vals[c])) for c in same_sign}
        best = min(dist.values())
        cands = [c for c in same_sign if dist[c] == best]          # nearest magnitude
        if len(cands) > 1:
            cands = [c for c in cands if c % 2 == 0]                # tie: even mantissa
        assert cands == [got], (x, got, cands)


def test_round_trip_and_monotone():
    vals = F8.e4m3_table()
    codes = np.array([c for c in range(256) if not math.isnan(vals[c])], dtype=np.uint8)
    assert np.array_equal(F8.quantize_e4m3(F8.decode_e4m3(codes).astype(np.float32), 1.0), codes)
    assert np.all(np.diff(vals[:0x7F]) > 0)
    assert np.array_equal(vals[0x80:0xFF], -vals[:0x7F])


def test_fp8_decode_equals_bf16_decode_on_exact_values():
    """Values drawn from the E4M3 table: quantising at scale 1 is lossless and
    bf16 holds the same numbers, so the two decode paths agree exactly."""
    rng = np.random.default_rng(11)
    nb, bs, Hkv, D, Hq, B = 12, 8, 2, 64, 4, 3
    vals = F8.e4m3_table()
    pool_codes = [c for c in range(256) if not math.isnan(vals[c]) and abs(vals[c]) <= 4]
    kc = rng.choice(pool_codes, (nb, bs, Hkv, D)).astype(np.uint8)
    vcodes = rng.choice(pool_codes, (nb, bs, Hkv, D)).astype(np.uint8)
    as_bf16 = lambda c: (F8.decode_e4m3(c).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    tables = rng.permutation(nb)[:B * 4].reshape(B, 4).astype(np.int32)
    lens = np.array([5, 17, 32], np.int32)
    q = (rng.standard_normal((B, Hq, D)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    o8, l8 = OA.paged_decode(q, kc, vcodes, tables, lens, 0.125, "bf16", "fp8", 1.0, 1.0)
    o16, l16 = OA.paged_decode(q, as_bf16(kc), as_bf16(vcodes), tables, lens, 0.125, "bf16")
    assert np.array_equal(o8, o16) and np.array_equal(l8, l16)
    # a scale multiplies every value: V scale scales the output, K scale the scores
    o8s, _ = OA.paged_decode(q, kc, vcodes, tables, lens, 0.125, "bf16", "fp8", 1.0, 0.5)
    assert np.allclose(o8s, 0.5 * o16, rtol=0, atol=1e-15)
    o8k, _ = OA.paged_decode(q, kc, vcodes, tables, lens, 0.25, "bf16", "fp8", 0.5, 1.0)
    assert np.allclose(o8k, o16, rtol=1e-13, atol=1e-13)


def test_planted_bias_mistake_fails_the_pins(monkeypatch):
    """Mutant: exponent bias 8 instead of 7 in the value table."""
    wrong = np.array([F8.e4m3_value(c) / 2 for c in range(256)])
    monkeypatch.setattr(F8, "_TABLE", wrong)
    monkeypatch.setattr(F8, "_POS_VALS", wrong[:0x7F])
    assert not _same(F8.decode_e4m3(np.array([0x38], np.uint8))[0], 1.0)
    x = _finite_bf16_in_range()
    assert not np.array_equal(F8.quantize_e4m3(x, 1.0), _torch_codes(x))
