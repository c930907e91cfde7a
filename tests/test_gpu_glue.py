"""GPU parity of the decode-stack glue kernels (bf16 -> fp32, RMSNorm,
residual add, bf16 head, argmax) against the oracle's definitions."""

import numpy as np
import pytest
import torch

import swiglu_decode_amd as sgd
import synth
from oracle import ref
from oracle.fp8 import f64_to_bf16_bits
from synth import bf16_to_f64
from tests.gpu_util import bf16_bits, dev, note

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("M,dd", [(1, 128), (5, 384), (64, 2560)])
def test_rmsnorm_and_residual(M, dd):
    d = dev()
    note(f"rmsnorm/residual M={M} d={dd}")
    rng = np.random.default_rng(7 + M)
    h = (rng.standard_normal((M, dd)) * 3.0).astype(np.float32)
    ht = torch.from_numpy(h).to(d)
    xb = sgd.rmsnorm_bf16(ht, 1e-6)
    torch.cuda.synchronize()
    want = f64_to_bf16_bits(ref.rmsnorm(h.astype(np.float64)))
    got = bf16_bits(xb)
    # the fp32 sum of squares differs from fp64 in its last bits: at most one
    # bf16 step, on a small fraction of elements
    diff = np.abs(got.astype(np.int32) - want.astype(np.int32))
    assert diff.max() <= 1 and np.mean(diff != 0) < 0.01, (diff.max(), np.mean(diff != 0))
    y = synth.random_bf16((M, dd), 9 + M, 1.0)
    sgd.residual_add(ht, y.to(d))
    torch.cuda.synchronize()
    exp = (h.astype(np.float64) + bf16_to_f64(y)).astype(np.float32)  # one fp32 rounding
    assert np.array_equal(ht.cpu().numpy(), exp)
    f = sgd.bf16_to_f32(y.to(d))
    torch.cuda.synchronize()
    assert np.array_equal(f.cpu().numpy().astype(np.float64), bf16_to_f64(y))


@pytest.mark.parametrize("M,dd", [(1, 128), (5, 384), (64, 2560), (3, 8192)])
def test_residual_rmsnorm_equals_the_two_calls(M, dd):
    # one launch for h += y and the next block's RMSNorm: bit-identical to
    # residual_add followed by rmsnorm_bf16 (h and x)
    d = dev()
    note(f"residual+rmsnorm M={M} d={dd}")
    rng = np.random.default_rng(17 + M)
    h = torch.from_numpy((rng.standard_normal((M, dd)) * 3.0).astype(np.float32)).to(d)
    y = synth.random_bf16((M, dd), 19 + M, 1.0).to(d)
    h2 = h.clone()
    sgd.residual_add(h, y)
    x = sgd.rmsnorm_bf16(h, 1e-6)
    x2 = sgd.residual_rmsnorm_bf16(h2, y, 1e-6)
    torch.cuda.synchronize()
    assert torch.equal(h2, h)
    assert torch.equal(bf16_bits_t(x2), bf16_bits_t(x))


def bf16_bits_t(t):
    return t.view(torch.int16)


@pytest.mark.parametrize("M,K,N", [(1, 128, 128), (17, 384, 256), (64, 2560, 4096)])
def test_head_logits(M, K, N):
    d = dev()
    note(f"head M={M} K={K} N={N}")
    rng = np.random.default_rng(11 + M)
    h = rng.standard_normal((M, K)).astype(np.float32)
    w = synth.random_bf16((N, K), 13 + N, 0.02)
    lg = sgd.head_logits(torch.from_numpy(h).to(d), w.to(d))
    torch.cuda.synchronize()
    want = ref.head_logits(h.astype(np.float64), bf16_to_f64(w))
    got = lg.cpu().numpy().astype(np.float64)
    # fp32 accumulation of K exact bf16 products
    err = np.max(np.abs(got - want)) / np.max(np.abs(want))
    assert err < 1e-5, err


def test_argmax_rows_ties_take_lowest_index():
    d = dev()
    note("argmax")
    rng = np.random.default_rng(5)
    lg = rng.standard_normal((9, 5000)).astype(np.float32)
    lg[1, 17] = lg[1, 4000] = 50.0          # tie: lowest index wins
    lg[2, :] = 1.0                          # all equal
    lg[3, 4999] = 99.0                      # last column
    lg[4, 0] = 99.0                         # first column
    lg[5, 10] = lg[5, 11] = lg[5, 12] = 7e3
    am = sgd.argmax_rows(torch.from_numpy(lg).to(d))
    torch.cuda.synchronize()
    assert np.array_equal(am.cpu().numpy(), ref.argmax_rows(lg))


def test_read_stream_runs_and_writes_nothing_but_the_sink():
    """The measurement aid reads its buffer and leaves it untouched."""
    d = dev()
    buf = torch.arange(1 << 20, dtype=torch.int32, device=d)
    ref_copy = buf.clone()
    sink = torch.full((1,), 7, dtype=torch.int32, device=d)
    sgd.read_stream(buf, sink)
    torch.cuda.synchronize()
    assert torch.equal(buf, ref_copy)
    with pytest.raises(Exception):
        sgd.read_stream(buf[1:])  # 4 bytes off the 16-byte alignment
