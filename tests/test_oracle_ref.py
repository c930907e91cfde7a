"""Pins of the oracle's fp64 GEMM / SwiGLU MLP / RMSNorm / stack: exact
integer arithmetic, identity-quantization special cases, closed forms and
brute-force loops."""

import math
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import fp8, quant, ref


def _bf16(rng, shape, std):
    return fp8.to_bf16((rng.standard_normal(shape) * std).astype(np.float32).astype(np.float64))


@pytest.mark.parametrize("fmt", ["block", "mx"])
def test_gemm_exact_rational_check(fmt):
    rng = np.random.default_rng(0)
    M, N, K = 3, 16 if fmt == "mx" else 128, 256
    x = _bf16(rng, (M, K), 1.0)
    w = _bf16(rng, (N, K), 0.02)
    xq, xs = quant.quantize_act(x, fmt)
    wq, ws = quant.quantize_weight(w, fmt)
    y = ref.gemm_quantized(xq, xs, wq, ws, fmt)
    xv = fp8.e4m3_decode(xq)
    wv = fp8.e4m3_decode(wq)
    g = 128 if fmt == "block" else 32
    for m in range(M):
        for n in range(0, N, 5):
            tot = Fraction(0)
            mag = 0.0
            for kb in range(K // g):
                if fmt == "block":
                    sc = Fraction(float(xs[m, kb])) * Fraction(float(ws[n // 128, kb]))
                else:
                    sc = Fraction(2) ** (int(xs[m, kb]) - 127) * Fraction(2) ** (int(ws[n, kb]) - 127)
                acc = sum(Fraction(xv[m, k]) * Fraction(wv[n, k]) for k in range(kb * g, kb * g + g))
                tot += sc * acc
                mag += float(sc) * float(sum(abs(Fraction(xv[m, k]) * Fraction(wv[n, k]))
                                             for k in range(kb * g, kb * g + g)))
            # float64 summation error bound: K * 2^-53 * sum of |terms|
            assert abs(float(tot) - y[m, n]) <= K * 2.0 ** -53 * mag


def test_gemm_identity_quantization_equals_textbook_matmul():
    # Operands already on the E4M3 grid with every group's amax at 448 quantize
    # to themselves with scale 1 (block) -> the scaled GEMM is the plain matmul.
    rng = np.random.default_rng(1)
    grid = fp8.e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    M, N, K = 4, 128, 256
    x = rng.choice(grid, (M, K)) * rng.choice([-1.0, 1.0], (M, K))
    w = rng.choice(grid, (N, K)) * rng.choice([-1.0, 1.0], (N, K))
    x[:, ::128] = 448.0
    w[::128, ::128] = 448.0
    w[1::128, 1::128] = 448.0
    for fmt in ("block",):
        xq, xs = quant.quantize_act(x, fmt)
        wq, ws = quant.quantize_weight(w, fmt)
        assert np.all(xs == 1.0) and np.all(ws == 1.0)
        y = ref.gemm_quantized(xq, xs, wq, ws, fmt)
        want = np.array([[sum(int(x[m, k] * 512) * int(w[n, k] * 512) for k in range(K))
                          for n in range(N)] for m in range(M)], dtype=np.float64) / 2.0 ** 18
        assert np.array_equal(y, want)


def test_gemm_mx_identity_quantization():
    # MX: a block whose amax lies in [256, 512) has X = 0 (scale 1).
    rng = np.random.default_rng(2)
    grid = fp8.e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    M, N, K = 2, 16, 128
    x = rng.choice(grid, (M, K))
    w = rng.choice(grid, (N, K)) * rng.choice([-1.0, 1.0], (N, K))
    x[:, ::32] = 320.0
    w[:, ::32] = -256.0
    xq, xs = quant.quantize_act(x, "mx")
    wq, ws = quant.quantize_weight(w, "mx")
    assert np.all(xs == 127) and np.all(ws == 127)
    y = ref.gemm_quantized(xq, xs, wq, ws, "mx")
    assert np.array_equal(y, x @ w.T)


def test_scaled_gemm_brute_force_loops():
    rng = np.random.default_rng(3)
    M, N, K = 2, 128, 128
    x = _bf16(rng, (M, K), 1.0)
    w = _bf16(rng, (N, K), 0.02)
    for fmt in ("block", "mx"):
        qw = ref.QWeight(w, fmt)
        y = ref.scaled_gemm(x, qw)
        xq, xs = quant.quantize_act(x, fmt)
        xd = quant.dequantize_act(xq, xs, fmt)
        wd = qw.deq()
        for m in range(M):
            for n in range(0, N, 3):
                s = 0.0
                for k in range(K):
                    s += xd[m, k] * wd[n, k]
                assert abs(s - y[m, n]) <= 1e-12 * (abs(s) + 1e-6)


def test_quantized_gemm_close_to_unquantized_within_fp8_error():
    rng = np.random.default_rng(4)
    x = _bf16(rng, (8, 1024), 1.0)
    w = _bf16(rng, (256, 1024), 0.02)
    for fmt in ("block", "mx"):
        y = ref.scaled_gemm(x, ref.QWeight(w, fmt))
        e = ref.rel_fro(y, x @ w.T)
        # E4M3 relative rounding error is at most 2^-4 per element, ~3% rms
        assert 0.005 < e < 0.08, (fmt, e)


def test_silu_closed_forms():
    assert ref.silu(0.0) == 0.0
    xs = np.linspace(-30, 30, 601)
    # silu(x) - silu(-x) = x * (sigmoid(x) + sigmoid(-x)) = x
    assert np.allclose(ref.silu(xs) - ref.silu(-xs), xs, rtol=0, atol=1e-12)
    # silu(x) = x / 2 * (1 + tanh(x / 2))
    # (the tanh form cancels for negative x, hence the absolute slack)
    assert np.allclose(ref.silu(xs), xs / 2 * (1 + np.tanh(xs / 2)), rtol=1e-13, atol=1e-13)
    assert ref.silu(-1000.0) == 0.0 and ref.silu(1000.0) == 1000.0
    assert abs(float(ref.silu(1.0)) - 1.0 / (1.0 + math.exp(-1.0))) < 1e-16


@pytest.mark.parametrize("fmt", ["block", "mx"])
def test_swiglu_mlp_brute_force_loops(fmt):
    rng = np.random.default_rng(5)
    M, d, F = 2, 128, 256
    x = _bf16(rng, (M, d), 1.0)
    wg = _bf16(rng, (F, d), 0.02)
    wu = _bf16(rng, (F, d), 0.02)
    wd = _bf16(rng, (d, F), 0.02)
    qg, qu, qd = (ref.QWeight(w, fmt) for w in (wg, wu, wd))
    out = ref.swiglu_mlp(x, qg, qu, qd, return_all=True)
    xq, sx = quant.quantize_act(x, fmt)
    xd = quant.dequantize_act(xq, sx, fmt)
    G, U, D = qg.deq(), qu.deq(), qd.deq()
    a = np.zeros((M, F))
    for m in range(M):
        for f in range(F):
            g = sum(xd[m, k] * G[f, k] for k in range(d))
            u = sum(xd[m, k] * U[f, k] for k in range(d))
            a[m, f] = g / (1.0 + math.exp(-g)) * u
    a32 = a.astype(np.float32).astype(np.float64)
    assert np.allclose(a, out["a"], rtol=1e-12, atol=1e-18)
    aq, sa = quant.quantize_act(a32, fmt)
    assert np.array_equal(aq, out["aq"])
    ad = quant.dequantize_act(aq, sa, fmt)
    for m in range(M):
        for n in range(0, d, 7):
            y = sum(ad[m, f] * D[n, f] for f in range(F))
            assert abs(y - out["y"][m, n]) <= 1e-12 * (abs(y) + 1e-9)


def test_swiglu_mlp_close_to_unquantized():
    rng = np.random.default_rng(6)
    x = _bf16(rng, (4, 256), 1.0)
    wg = _bf16(rng, (512, 256), 0.02)
    wu = _bf16(rng, (512, 256), 0.02)
    wd = _bf16(rng, (256, 512), 0.02)
    y0 = ref.swiglu_mlp_unquantized(x, wg, wu, wd)
    for fmt in ("block", "mx"):
        y = ref.swiglu_mlp(x, *(ref.QWeight(w, fmt) for w in (wg, wu, wd)))
        e = ref.rel_fro(y, y0)
        assert 0.005 < e < 0.15, (fmt, e)


def test_rmsnorm_closed_forms():
    h = np.full((2, 64), 3.0)
    h[1] = -0.5
    r = ref.rmsnorm(h, eps=0.0)
    assert np.allclose(r[0], 1.0) and np.allclose(r[1], -1.0)
    r = ref.rmsnorm(h, eps=1e-6)
    assert np.allclose(r[0], 3.0 / math.sqrt(9.0 + 1e-6), rtol=1e-15)
    rng = np.random.default_rng(7)
    h = rng.standard_normal((4, 2560)) * 10
    r = ref.rmsnorm(h, eps=0.0)
    assert np.allclose(np.mean(r * r, axis=1), 1.0, rtol=1e-12)
    assert np.allclose(ref.rmsnorm(7.5 * h, eps=0.0), r, rtol=1e-12)


def test_stack_layer_and_head_rounding_points():
    rng = np.random.default_rng(8)
    M, d, F, V = 4, 128, 256, 64
    h = _bf16(rng, (M, d), 1.0)
    ws = [_bf16(rng, s, 0.02) for s in ((F, d), (F, d), (d, F))]
    q = [ref.QWeight(w, "block") for w in ws]
    h1 = ref.stack_layer(h, *q)
    xl = fp8.to_bf16(ref.rmsnorm(h))
    y = fp8.to_bf16(ref.swiglu_mlp(xl, *q))
    assert np.array_equal(h1, (h + y).astype(np.float32).astype(np.float64))
    assert np.array_equal(fp8.to_bf16(y), y)
    head = _bf16(rng, (V, d), 0.02)
    lg = ref.head_logits(h1, head)
    assert np.allclose(lg, fp8.to_bf16(h1) @ head.T, rtol=0, atol=0)


def test_argmax_lowest_index_on_ties():
    lg = np.array([[1.0, 3.0, 3.0, 0.0], [5.0, 5.0, 5.0, 5.0]])
    assert ref.argmax_rows(lg).tolist() == [1, 0]


def test_error_metrics():
    r = np.array([[3.0, 4.0]])
    assert ref.rel_fro(r, r) == 0.0
    assert ref.rel_fro(np.array([[3.0, 4.0 + 5.0]]), r) == 1.0
    assert ref.max_abs_ratio(np.array([[3.0, 4.4]]), r) == pytest.approx(0.1)


# ---------------------------------------------------------------------------
# Hand-worked decode-stack examples (tests/golden/stack_worked_example.txt,
# which derives every value in its comments)
# ---------------------------------------------------------------------------
def _golden(name):
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", name)
    vals = {}
    for line in open(path):
        line = line.strip()
        if line and not line.startswith("#"):
            k, v = line.split(":", 1)
            vals[k.strip()] = [float(t) for t in v.split()]
    return vals


def test_stack_layer_worked_example():
    g = _golden("stack_worked_example.txt")
    x = np.empty(128)
    x[0:4] = 1.75
    x[4:117] = [(-1.0) ** i for i in range(4, 117)]
    x[117:] = 0.5
    h = (2.0 * x)[None, :]
    wg = np.zeros((128, 128))
    wg[np.arange(127), np.arange(127)] = 1.0
    wg[127, 127] = 448.0
    wg[0, 5] = 0.25
    wu = np.zeros((128, 128))
    wu[0, 3] = 448.0
    wd = np.zeros((128, 128))
    wd[0:5, 0] = [448.0, 1.0, -0.5, 2.0 ** -9, -3.5]
    out = ref.stack_layer(h, *(ref.QWeight(w, "block") for w in (wg, wu, wd)), eps=0.0)
    assert out[0, :5].tolist() == g["ex1_h_out_0_4"]
    assert np.array_equal(out[0, 5:], h[0, 5:])


@pytest.mark.parametrize("fmt", ["block", "mx"])
def test_stack_layer_zero_weights_rounds_the_residual_to_fp32(fmt):
    g = _golden("stack_worked_example.txt")
    h = np.ones((1, 128))
    h[0, :4] = [1.0 + 2.0 ** -30, 3.0 + 2.0 ** -24, -(2.0 + 3.0 * 2.0 ** -23), 0.75 * 2.0 ** -149]
    z = [ref.QWeight(np.zeros(s), fmt) for s in ((128, 128), (128, 128), (128, 128))]
    out = ref.stack_layer(h, *z)
    assert out[0, :4].tolist() == g["ex2_h_out_0_3"]
    assert np.array_equal(out[0, 4:], h[0, 4:])


def test_head_logits_worked_example():
    g = _golden("stack_worked_example.txt")
    h = np.array([[1.0 + 2.0 ** -9, 1.0 + 3.0 * 2.0 ** -8, -(2.0 + 2.0 ** -7), 0.5],
                  [2.0 ** -130, 7.0, 255.5, 1.0 / 3.0]])
    w = np.array([[1.0, 0, 0, 0], [1, 1, 1, 1], [0.5, -1, 2, 3], [0, 2, 0, 0]])
    lg = ref.head_logits(h, w)
    assert lg[0].tolist() == g["ex3_logits_0"]
    assert lg[1].tolist() == g["ex3_logits_1"]
    assert ref.argmax_rows(lg).tolist() == [int(v) for v in g["ex3_argmax"]]
