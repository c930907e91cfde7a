"""Pins of the oracle's E4M3 / UE8M0 / bf16 codecs against the OCP
definitions, brute force and torch's independent implementations."""

import math
import os

import numpy as np
import pytest
import torch

from oracle import fp8

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _finite_codes():
    return np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)


def test_decode_matches_ocp_pin_file():
    n = 0
    for line in open(os.path.join(GOLDEN, "e4m3_ocp_pins.txt")):
        line = line.split("#")[0].strip()
        if not line:
            continue
        code, val = line.split()
        got = fp8.e4m3_decode(np.uint8(int(code, 16)))
        if val == "nan":
            assert np.isnan(got)
        else:
            assert got == float(val)
            assert np.signbit(got) == val.startswith("-")
        n += 1
    assert n >= 15


def test_decode_matches_torch_for_all_codes():
    t = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    ours = fp8.e4m3_decode(np.arange(256, dtype=np.uint8))
    both_nan = np.isnan(t) & np.isnan(ours)
    assert np.all(both_nan | (t == ours))
    assert np.array_equal(np.signbit(t[~both_nan]), np.signbit(ours[~both_nan]))
    assert int(np.isnan(ours).sum()) == 2


def test_positive_codes_are_monotone_and_uniform_below_min_normal():
    v = fp8.e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    assert np.all(np.diff(v) > 0)
    assert np.allclose(np.diff(v[:9]), 2.0 ** -9, rtol=0, atol=0)
    assert v[-1] == 448.0


def test_encode_decode_roundtrip_all_finite_codes():
    codes = _finite_codes()
    assert codes.size == 254
    assert np.array_equal(fp8.e4m3_encode(fp8.e4m3_decode(codes)), codes)


def _brute_encode(x):
    """Nearest finite E4M3 value by exhaustive search; ties to the even code;
    saturation at 448; NaN -> 0x7F with sign; sign of zero kept."""
    x = np.asarray(x, dtype=np.float64)
    pos = np.arange(0x7F, dtype=np.uint8)            # 0x00..0x7E
    vals = fp8.e4m3_decode(pos)
    a = np.abs(x)
    out = np.empty(x.shape, dtype=np.uint8)
    for s in range(0, x.size, 1 << 16):
        aa = a[s:s + (1 << 16)]
        d = np.abs(aa[:, None] - vals[None, :])
        dmin = d.min(axis=1, keepdims=True)
        cand = d == dmin
        # among tied candidates prefer even codes; with two ties exactly one is even
        even = cand & ((pos[None, :] & 1) == 0)
        pick = np.where(even.any(axis=1), even.argmax(axis=1), cand.argmax(axis=1))
        out[s:s + (1 << 16)] = pos[pick]
    out = np.where(a >= 448.0, np.uint8(0x7E), out)
    out = np.where(np.isnan(x), np.uint8(0x7F), out)
    return (out | (np.signbit(x).astype(np.uint8) << 7)).astype(np.uint8)


def test_encode_midpoints_tie_to_even_and_neighbours_round_nearer():
    v = fp8.e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    for c in range(0x7E):
        mid = (v[c] + v[c + 1]) / 2.0  # exact in float64
        even = c if c % 2 == 0 else c + 1
        assert fp8.e4m3_encode(mid) == even, hex(c)
        assert fp8.e4m3_encode(-mid) == (even | 0x80)
        lo = float(np.nextafter(np.float32(mid), np.float32(0)))
        hi = float(np.nextafter(np.float32(mid), np.float32(1e9)))
        assert fp8.e4m3_encode(lo) == c
        assert fp8.e4m3_encode(hi) == c + 1


def test_encode_brute_force_all_bf16_patterns():
    bits = np.arange(65536, dtype=np.uint16)
    x = fp8.bf16_bits_to_f64(bits)
    assert np.array_equal(fp8.e4m3_encode(x), _brute_encode(x))


def test_encode_brute_force_random_fp32():
    rng = np.random.default_rng(7)
    n = 1_000_000
    mag = np.exp2(rng.uniform(-14, 10, n))
    x = (mag * rng.choice([-1.0, 1.0], n)).astype(np.float32).astype(np.float64)
    assert np.array_equal(fp8.e4m3_encode(x), _brute_encode(x))


def test_encode_matches_torch_cast_below_464():
    # torch's cast is RNE but does not saturate, so compare only |v| < 464.
    rng = np.random.default_rng(11)
    x = np.concatenate([
        fp8.bf16_bits_to_f64(np.arange(65536, dtype=np.uint16)),
        (np.exp2(rng.uniform(-16, 9, 2_000_000)) * rng.choice([-1.0, 1.0], 2_000_000)),
    ]).astype(np.float32)
    x = x[np.isfinite(x) & (np.abs(x) < 464)]
    t = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(fp8.e4m3_encode(x.astype(np.float64)), t)


def test_encode_saturates_and_keeps_signs():
    enc = lambda v: int(fp8.e4m3_encode(np.float64(v)))
    for v in (448.0, 449.0, 463.99, 464.0, 480.0, 1e6, 3.4e38, math.inf):
        assert enc(v) == 0x7E and enc(-v) == 0xFE
    assert enc(0.0) == 0x00 and enc(-0.0) == 0x80
    assert enc(-1e-10) == 0x80 and enc(2.0 ** -10) == 0x00
    assert enc(1.5 * 2.0 ** -10) == 0x01       # rounds up to the min subnormal
    assert enc(math.nan) == 0x7F
    assert enc(-math.nan) == 0xFF


def test_ue8m0_decode_and_torch_e8m0():
    e = np.arange(256)
    v = fp8.ue8m0_decode(e)
    assert v[127] == 1.0 and v[0] == 2.0 ** -127 and v[254] == 2.0 ** 127
    assert np.isnan(v[255])
    t = torch.arange(256, dtype=torch.uint8).view(torch.float8_e8m0fnu).double().numpy()
    ok = (t == v) | (np.isnan(t) & np.isnan(v))
    assert ok.all()


def test_floor_log2_exact_including_subnormals():
    rng = np.random.default_rng(3)
    x = np.concatenate([np.exp2(rng.uniform(-149, 127, 100000)).astype(np.float32),
                        np.float32(2.0) ** np.arange(-149, 128, dtype=np.float32)])
    x = x[x > 0].astype(np.float64)
    want = np.array([math.frexp(float(a))[1] - 1 for a in x])
    assert np.array_equal(fp8.floor_log2(x), want)


def test_to_bf16_matches_torch_on_fp32_inputs():
    rng = np.random.default_rng(5)
    x = np.concatenate([
        rng.standard_normal(500000).astype(np.float32) * np.float32(3.0),
        np.exp2(rng.uniform(-140, 127, 200000)).astype(np.float32),
        np.array([0.0, -0.0, 1.0, 65504.0, 3.3e38, 1e-40], dtype=np.float32),
    ])
    want = torch.from_numpy(x).to(torch.bfloat16).double().numpy()
    got = fp8.to_bf16(x.astype(np.float64))
    assert np.array_equal(got, want)
    assert np.array_equal(np.signbit(got), np.signbit(want))


def test_to_bf16_single_rounding_from_float64():
    # 1 + 2^-8 is the midpoint between bf16 neighbours 1 and 1 + 2^-7; a value
    # a hair above it must round up (a detour through fp32 would lose the hair
    # and round to even, i.e. down).
    v = 1.0 + 2.0 ** -8 + 2.0 ** -40
    assert fp8.to_bf16(v) == 1.0 + 2.0 ** -7
    assert fp8.to_bf16(1.0 + 2.0 ** -8) == 1.0
    assert fp8.to_bf16(1.0 + 3 * 2.0 ** -8) == 1.0 + 2.0 ** -6


def test_bf16_bits_roundtrip():
    bits = np.arange(65536, dtype=np.uint16)
    v = fp8.bf16_bits_to_f64(bits)
    fin = np.isfinite(v)
    assert np.array_equal(fp8.f64_to_bf16_bits(v[fin]), bits[fin])
