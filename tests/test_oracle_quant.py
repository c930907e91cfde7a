"""Pins of the oracle's block-128 / MX-32 quantizers: hand-worked examples,
exact rational arithmetic, invariants and brute force."""

import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import fp8, quant
from oracle.fp8 import bf16_bits_to_f64

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _fraction_to_f32(q: Fraction) -> float:
    """Round an exact rational to the nearest fp32 value, ties to even, by
    exact comparison with its two fp32 neighbours (normal range)."""
    lo = np.float32(float(q))  # within one fp32 ulp of q
    cands = {float(lo), float(np.nextafter(lo, np.float32(np.inf))),
             float(np.nextafter(lo, np.float32(-np.inf)))}
    best = None
    for c in sorted(cands):
        d = abs(Fraction(c) - q)
        if best is None or d < best[0]:
            best = (d, c)
        elif d == best[0]:
            # tie: the even significand
            m_c = np.float32(c).view(np.uint32) & 1
            if m_c == 0:
                best = (d, c)
    return best[1]


def _load_worked():
    rows = []
    for line in open(os.path.join(GOLDEN, "quant_worked_examples.txt")):
        line = line.split("#")[0].strip()
        if not line:
            continue
        fields = line.split()
        kv = dict(f.split("=") for f in fields[1:])
        rows.append((fields[0], kv))
    return rows


def test_worked_examples_from_golden_file():
    rows = _load_worked()
    assert len(rows) >= 5
    for fmt, kv in rows:
        vals = [float(v) for v in kv["in"].split(",")]
        want = [int(c, 16) for c in kv["codes"].split(",")]
        size = quant.BLOCK if fmt == "block" else quant.MX
        x = np.zeros((1, size))
        x[0, :len(vals)] = vals
        codes, s = quant.quantize_act(x, fmt)
        assert list(codes[0, :len(vals)]) == want, (fmt, kv)
        if fmt == "block":
            assert float(s[0, 0]) == float(kv["scale"])
        else:
            assert int(s[0, 0]) == int(kv["scale_e8m0"], 16)


def _rand_bf16(rng, shape, std=1.0):
    x = (rng.standard_normal(shape) * std).astype(np.float32)
    return fp8.to_bf16(x.astype(np.float64))


def test_block_scale_is_correctly_rounded_quotient():
    rng = np.random.default_rng(1)
    amax = np.abs(_rand_bf16(rng, 3000, 5.0)) + 0.0
    amax = amax[amax > 0]
    s = quant.block_scale(amax)
    for a, sv in zip(amax[:3000], s[:3000]):
        assert float(sv) == _fraction_to_f32(Fraction(float(a)) / 448)


def test_block_codes_are_encode_of_correctly_rounded_division():
    rng = np.random.default_rng(2)
    x = _rand_bf16(rng, (4, 256), 2.0)
    codes, s = quant.quantize_act(x, "block")
    for m in range(4):
        for k in range(0, 256, 7):
            q = _fraction_to_f32(Fraction(float(x[m, k])) / Fraction(float(s[m, k // 128])))
            assert codes[m, k] == fp8.e4m3_encode(q)


def test_block_invariants_random_groups():
    rng = np.random.default_rng(3)
    x = _rand_bf16(rng, (64, 1024), 1.0)
    codes, s = quant.quantize_act(x, "block")
    mag = codes & 0x7F
    assert mag.max() <= 0x7E
    g = np.abs(x.reshape(64, 8, 128))
    arg = g.argmax(axis=2)
    amax_codes = np.take_along_axis(mag.reshape(64, 8, 128), arg[:, :, None], 2)
    assert np.all(amax_codes == 0x7E)
    # per-element error <= half the E4M3 spacing at |v|/s, times s
    deq = quant.dequantize_act(codes, s, "block")
    r = np.abs(x) / np.repeat(s.astype(np.float64), 128, axis=1)
    e = np.maximum(np.floor(np.log2(np.maximum(r, 2.0 ** -6))), -6)
    half = 0.5 * np.exp2(e - 3) * np.repeat(s.astype(np.float64), 128, axis=1)
    assert np.all(np.abs(deq - x) <= half * (1 + 2.0 ** -20))


def test_block_power_of_two_scaling_is_exact_metamorphic():
    rng = np.random.default_rng(4)
    x = _rand_bf16(rng, (8, 512), 1.0)
    c0, s0 = quant.quantize_act(x, "block")
    for k in (-20, -3, 1, 7, 30):
        c1, s1 = quant.quantize_act(x * 2.0 ** k, "block")
        assert np.array_equal(c0, c1)
        assert np.array_equal(s1.astype(np.float64), s0.astype(np.float64) * 2.0 ** k)


def test_block_zero_group_gives_unit_scale():
    x = np.zeros((2, 256))
    x[1, 128:] = -0.0
    x[0, 5] = -0.0
    codes, s = quant.quantize_act(x, "block")
    assert np.all(s == 1.0)
    assert codes[0, 5] == 0x80 and codes[0, 4] == 0x00


def test_block_weight_tiles_use_tile_amax():
    rng = np.random.default_rng(6)
    w = _rand_bf16(rng, (256, 384), 0.02)
    w[130, 300] = 5.0  # tile (1, 2)
    codes, s = quant.quantize_weight(w, "block")
    assert s.shape == (2, 3)
    tile_amax = np.abs(w.reshape(2, 128, 3, 128)).max(axis=(1, 3))
    assert np.array_equal(s, quant.block_scale(tile_amax))
    assert codes[130, 300] == 0x7E
    deq = quant.dequantize_weight(codes, s, "block")
    assert np.max(np.abs(deq - w)) <= 5.0 / 448 * 16  # coarse sanity


def test_mx_scale_invariants_and_brute_force_exponent():
    bits = np.arange(1, 0x7F80, dtype=np.uint16)  # all positive finite bf16
    amax = bf16_bits_to_f64(bits)
    X = quant.mx_scale_exponent(amax)
    # brute force: the largest X with amax * 2^-X >= 256 (i.e. in [256, 512))
    lo = np.floor(np.log2(amax)).astype(np.int64) - 12
    best = np.full(amax.shape, -10**9)
    for off in range(0, 16):
        cand = lo + off
        ok = np.ldexp(amax, (-cand).astype(np.int32)) >= 256
        best = np.where(ok, cand, best)
    want = np.clip(best, -127, 127)
    assert np.array_equal(X, want)
    unclamped = best >= -127
    r = np.ldexp(amax[unclamped], (-X[unclamped]).astype(np.int32))
    assert np.all((r >= 256) & (r < 512))


def test_mx_quantization_codes_and_scales():
    rng = np.random.default_rng(8)
    x = _rand_bf16(rng, (16, 512), 3.0)
    codes, e = quant.quantize_act(x, "mx")
    assert e.dtype == np.uint8 and e.shape == (16, 16)
    # the amax element of each block encodes into 0x78..0x7E
    g = np.abs(x.reshape(16, 16, 32))
    arg = g.argmax(axis=2)
    mag = (codes & 0x7F).reshape(16, 16, 32)
    am = np.take_along_axis(mag, arg[:, :, None], 2)
    assert np.all((am >= 0x78) & (am <= 0x7E))
    # scale is exactly 2^(E-127) and deq = decode(code) * scale
    deq = quant.dequantize_act(codes, e, "mx")
    want = fp8.e4m3_decode(codes).reshape(16, 16, 32) * np.exp2(e.astype(np.float64) - 127)[:, :, None]
    assert np.array_equal(deq, want.reshape(16, 512))
    # metamorphic: x * 2^k -> E + k, identical codes
    for k in (-5, 3, 40):
        c1, e1 = quant.quantize_act(x * 2.0 ** k, "mx")
        assert np.array_equal(c1, codes)
        assert np.array_equal(e1.astype(int), e.astype(int) + k)


def test_mx_zero_block_and_saturation():
    x = np.zeros((1, 64))
    x[0, 32] = 480.0   # floor(log2 480) = 8 -> X = 0, 480 saturates to 448
    x[0, 33] = -500.0  # bf16-exact? 500 = 1.953125 * 2^8 -> 8 bits -> yes
    codes, e = quant.quantize_act(x, "mx")
    assert e[0, 0] == 0 and np.all(codes[0, :32] == 0)
    assert e[0, 1] == 127 and codes[0, 32] == 0x7E and codes[0, 33] == 0xFE


def test_mx_weight_is_rowwise_1x32():
    rng = np.random.default_rng(9)
    w = _rand_bf16(rng, (32, 256), 0.02)
    c, e = quant.quantize_weight(w, "mx")
    c2, e2 = quant.quantize_act(w, "mx")
    assert np.array_equal(c, c2) and np.array_equal(e, e2)
    assert e.shape == (32, 8)


def test_transposed_scale_layout_is_a_large_error():
    # The failure class the pages describe (a scale-stride mix-up that keeps
    # full speed but corrupts results) must show up as a large error, not a
    # subtle one: dequantize with the block-scale grid transposed.
    rng = np.random.default_rng(10)
    # tile magnitudes differ by powers of two in a non-symmetric pattern
    tile_exp = np.array([[0, 3], [-4, 1]])
    mult = np.exp2(np.kron(tile_exp, np.ones((128, 128))))
    w = fp8.to_bf16(rng.standard_normal((256, 256)) * 0.02 * mult)
    c, s = quant.quantize_weight(w, "block")
    good = quant.dequantize_weight(c, s, "block")
    bad = quant.dequantize_weight(c, s.T.copy(), "block")
    err_good = np.linalg.norm(good - w) / np.linalg.norm(w)
    err_bad = np.linalg.norm(bad - w) / np.linalg.norm(w)
    assert err_good < 0.05 and err_bad > 0.3
