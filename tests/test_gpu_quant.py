"""GPU parity of quantize/pack, unpack and activation quantization: bit-exact
against the oracle."""

import numpy as np
import pytest
import torch

import swiglu_decode_amd as sgd
import synth
from oracle import fp8, layout, quant
from synth import bf16_to_f64
from tests.gpu_util import dev, note

pytestmark = pytest.mark.gpu


def _weights_special(N, K, seed):
    """N(0, 0.02) weights with edge cases planted: an all-zero 128x128 tile,
    an all-zero 1x32 block, signed zeros, huge and tiny magnitudes, and exact
    e4m3 midpoints after scaling."""
    w = synth.random_bf16((N, K), seed, 0.02).float()
    w[N - 128:, K - 128:] = 0.0            # an all-zero 128x128 tile (if N or K >= 256)
    w[10, 64:96] = 0.0                     # an all-zero 1x32 block
    w[11, 96:128] = torch.tensor([2.0 ** -133 * (i + 1) for i in range(32)])  # subnormal-only block
    w[3, 5] = -0.0
    w[5, 7] = 3.0e38
    w[6, 9] = -1.0e-30
    w[7, 11] = 2.0 ** -130  # bf16 subnormal
    w[9, 0:32] = torch.tensor([448.0, 464.0, 480.0, -0.5] + [0.0] * 28)
    return w.to(torch.bfloat16)


SHAPES = [(128, 128), (256, 384), (384, 256), (128, 640), (512, 1152)]


@pytest.mark.parametrize("fmt", ["block", "mx"])
@pytest.mark.parametrize("N,K", SHAPES)
def test_pack_weight_bit_exact(fmt, N, K):
    d = dev()
    note(f"pack {fmt} {N}x{K}")
    w = _weights_special(N, K, 100 + N + K)
    pw = sgd.quantize_pack_weight(w.to(d), fmt)
    torch.cuda.synchronize()
    codes_ref, scales_ref = quant.quantize_weight(bf16_to_f64(w), fmt)
    packed_ref = layout.pack_codes(codes_ref)
    assert np.array_equal(pw.codes.cpu().numpy(), packed_ref)
    if fmt == "block":
        got = pw.scales.cpu().view(torch.float32).numpy().reshape(N // 128, K // 128)
        assert np.array_equal(got.view(np.uint32), scales_ref.astype(np.float32).view(np.uint32))
    else:
        assert np.array_equal(pw.scales.cpu().numpy(), layout.pack_mx_scales(scales_ref))
    # unpack (GPU) round trip to the logical layout
    c2, s2 = sgd.unpack_weight(pw)
    assert np.array_equal(c2.cpu().numpy(), codes_ref)
    if fmt == "block":
        assert np.array_equal(s2.cpu().numpy().view(np.uint32), scales_ref.astype(np.float32).view(np.uint32))
    else:
        assert np.array_equal(s2.cpu().numpy(), scales_ref)


@pytest.mark.parametrize("fmt", ["block", "mx"])
def test_pack_all_bf16_patterns(fmt):
    # every finite bf16 value appears in the weight, in tiles of varied amax
    d = dev()
    note(f"pack all-bf16 {fmt}")
    bits = np.arange(65536, dtype=np.uint16)
    vals = fp8.bf16_bits_to_f64(bits)
    vals = vals[np.isfinite(vals)]
    rng = np.random.default_rng(3)
    rng.shuffle(vals)
    K = 512
    N = (vals.size + K - 1) // K
    N = (N + 127) // 128 * 128
    buf = np.zeros(N * K)
    buf[:vals.size] = vals
    w = torch.from_numpy(buf.reshape(N, K).astype(np.float32)).to(torch.bfloat16)
    assert np.array_equal(bf16_to_f64(w), buf.reshape(N, K))
    pw = sgd.quantize_pack_weight(w.to(d), fmt)
    codes_ref, scales_ref = quant.quantize_weight(buf.reshape(N, K), fmt)
    assert np.array_equal(pw.codes.cpu().numpy(), layout.pack_codes(codes_ref))


@pytest.mark.parametrize("fmt", ["block", "mx"])
@pytest.mark.parametrize("M,K", [(1, 128), (3, 256), (16, 2048), (77, 640), (128, 4096)])
def test_quantize_act_bit_exact(fmt, M, K):
    d = dev()
    note(f"act quant {fmt} {M}x{K}")
    x = synth.random_bf16((M, K), 7 + M + K, 1.0).float()
    x[0, :128] = 0.0
    if M > 1:
        x[1, 3] = 1e30
        x[1, 4] = -1e-35
    x = x.to(torch.bfloat16)
    codes, scales = sgd.quantize_act(x.to(d), fmt)
    c_ref, s_ref = quant.quantize_act(bf16_to_f64(x), fmt)
    assert np.array_equal(codes.cpu().numpy(), c_ref)
    if fmt == "block":
        assert np.array_equal(scales.cpu().numpy().view(np.uint32), s_ref.view(np.uint32))
    else:
        assert np.array_equal(scales.cpu().numpy(), s_ref)


@pytest.mark.parametrize("fmt", ["block", "mx"])
def test_act_quant_of_every_bf16_value(fmt):
    d = dev()
    note(f"act quant all bf16 {fmt}")
    bits = np.arange(65536, dtype=np.uint16)
    vals = fp8.bf16_bits_to_f64(bits)
    vals = vals[np.isfinite(vals)]
    K = 1024
    M = (vals.size + K - 1) // K
    buf = np.zeros(M * K)
    buf[:vals.size] = vals
    x = torch.from_numpy(buf.reshape(M, K).astype(np.float32)).to(torch.bfloat16)
    codes, scales = sgd.quantize_act(x.to(d), fmt)
    c_ref, s_ref = quant.quantize_act(buf.reshape(M, K), fmt)
    assert np.array_equal(codes.cpu().numpy(), c_ref)
