"""GPU parity of the unfused pipeline (gate/up GEMM into fp32, standalone
SwiGLU + re-quantization, down GEMM from pre-quantized activations, with
the intermediates in HBM) and of its building blocks."""

import numpy as np
import pytest
import torch

import swiglu_decode_amd as sgd
import synth
from oracle import quant, ref
from synth import bf16_to_f64
from tests.gpu_util import assert_close, dev, gpu_out_f64, note, oracle_weight
from tests.test_gpu_internals import _mpad, mtile_codes, mtile_scales

pytestmark = pytest.mark.gpu


def to_mtile(codes, scales, fmt):
    """Logical (codes [M, K], scales) -> workspace layout bytes (inverse of
    tests.test_gpu_internals.mtile_codes / mtile_scales)."""
    M, K = codes.shape
    cb = np.empty(M * K, dtype=np.uint8)
    for t in range(0, M, 16):
        Mt = min(16, M - t)
        cb[t * K:t * K + Mt * K] = codes[t:t + Mt].reshape(Mt, K // 16, 16).transpose(1, 0, 2).reshape(-1)
    if fmt == "block":
        s = np.zeros((K // 128, _mpad(M)), dtype=np.float32)
        s[:, :M] = scales.T
        sb = s.view(np.uint8).reshape(-1)
    else:
        sb = np.empty(M * (K // 32), dtype=np.uint8)
        for t in range(0, M, 16):
            Mt = min(16, M - t)
            blk = scales[t:t + Mt].reshape(Mt, K // 128, 4).transpose(1, 0, 2).reshape(-1)
            sb[t * (K // 32):t * (K // 32) + blk.size] = blk
    return cb, sb


@pytest.mark.parametrize("fmt", ["block", "mx"])
def test_stacked_packing(fmt):
    d = dev()
    note(f"stack_packed {fmt}")
    a = synth.random_bf16((384, 640), 31, 0.02)
    b = synth.random_bf16((256, 640), 32, 0.02)
    pa, pb = sgd.quantize_pack_weight(a.to(d), fmt), sgd.quantize_pack_weight(b.to(d), fmt)
    pab = sgd.quantize_pack_weight(torch.cat([a, b]).to(d), fmt)
    st = sgd.stack_packed(pa, pb)
    torch.cuda.synchronize()
    assert (st.N, st.K) == (640, 640)
    assert torch.equal(st.codes, pab.codes) and torch.equal(st.scales, pab.scales)


@pytest.mark.parametrize("fmt", ["block", "mx"])
@pytest.mark.parametrize("M,N,K", [(1, 512, 1024), (16, 1024, 512), (33, 256, 640), (128, 512, 512)])
def test_gemm_f32_and_prequantized(fmt, M, N, K):
    """sgd_scaled_gemm_f32 rounds to the bf16 result of sgd_scaled_gemm bit for
    bit; sgd_scaled_gemm_q on the oracle's Q(x) (laid out by this test) gives
    the result of sgd_scaled_gemm on x: bit for bit where both read Q(x) from
    memory (M > 32), else up to the summation order (the bf16-input call
    keeps Q(x) in LDS and may run on a grid of another size)."""
    d = dev()
    note(f"gemm f32 / prequantized {fmt} M={M} N={N} K={K}")
    x = synth.random_bf16((M, K), 51 + M, 1.0)
    w = synth.random_bf16((N, K), 52 + N, 0.02)
    pw = sgd.quantize_pack_weight(w.to(d), fmt)
    y16 = sgd.scaled_gemm(x.to(d), pw)
    y32 = sgd.scaled_gemm_f32(x.to(d), pw)
    c, s = quant.quantize_act(bf16_to_f64(x), fmt)
    cb, sb = to_mtile(c, s, fmt)
    yq = sgd.scaled_gemm_q(torch.from_numpy(cb).to(d), torch.from_numpy(sb).to(d), M, pw)
    torch.cuda.synchronize()
    assert torch.equal(y32.to(torch.bfloat16), y16)
    if M > 32:
        assert torch.equal(yq, y16)
    else:
        assert ref.rel_fro(gpu_out_f64(yq), gpu_out_f64(y16)) <= 2e-3
    assert_close(gpu_out_f64(y32), ref.scaled_gemm(bf16_to_f64(x), oracle_weight(w, fmt)), f"gemm_f32 {fmt}")


@pytest.mark.parametrize("fmt", ["block", "mx"])
@pytest.mark.parametrize("M,F", [(1, 1024), (5, 3072), (16, 6144), (64, 2048), (128, 1024)])
def test_swiglu_quantize(fmt, M, F):
    """Q(silu(g) * u) against the oracle's quantizer applied to the fp64
    product rounded to fp32.  The kernel forms the product in fp32 (the
    fused kernel's arithmetic), a few ulps from fl32 of the fp64 one, so a
    code may move by one step where the product sits at an E4M3 rounding
    midpoint: at most 1 in 1000 codes, by one step."""
    d = dev()
    note(f"swiglu_quantize {fmt} M={M} ffn={F}")
    rng = np.random.default_rng(60 + M + F)
    gu = (rng.standard_normal((M, 2 * F)) * 3.0).astype(np.float32)
    aq, sc = sgd.swiglu_quantize(torch.from_numpy(gu).to(d), fmt)
    torch.cuda.synchronize()
    g, u = gu[:, :F].astype(np.float64), gu[:, F:].astype(np.float64)
    a32 = (ref.silu(g) * u).astype(np.float32).astype(np.float64)
    c_ref, s_ref = quant.quantize_act(a32, fmt)
    codes = mtile_codes(aq.cpu().numpy(), M, F)
    scales = mtile_scales(sc.cpu().numpy(), M, F, fmt)
    mism = codes != c_ref
    print(f"[parity] swiglu_quantize {fmt} M={M} ffn={F}: {int(mism.sum())} of {codes.size} codes differ",
          flush=True)
    assert mism.mean() <= 1e-3
    step = np.abs(codes.astype(np.int64) - c_ref.astype(np.int64))[mism]
    assert np.all(step == 1)
    if fmt == "block":
        np.testing.assert_allclose(scales, s_ref, rtol=1e-6)
        if M < _mpad(M):  # padded rows hold zero scales
            raw = sc.cpu().numpy().view(np.float32).reshape(F // 128, _mpad(M))
            assert np.all(raw[:, M:] == 0)
    else:
        assert np.mean(scales != s_ref) <= 1e-3


def _unfused(name, fmt, M, d):
    wl = synth.WORKLOADS[name]
    inp = synth.mlp_inputs(wl, M)
    pg, pu, pd = [sgd.quantize_pack_weight(inp[k].to(d), fmt) for k in ("wg", "wu", "wd")]
    x = inp["x"][:M].contiguous().to(d)
    y_u = sgd.unfused_swiglu_mlp(x, sgd.stack_packed(pg, pu), pd)
    y_f = sgd.fused_swiglu_mlp(x, pg, pu, pd)
    torch.cuda.synchronize()
    q = [oracle_weight(inp[k], fmt) for k in ("wg", "wu", "wd")]
    y_ref = ref.swiglu_mlp(bf16_to_f64(inp["x"][:M]), *q)
    assert_close(gpu_out_f64(y_u), y_ref, f"unfused {name} {fmt} M={M}")
    rf = ref.rel_fro(gpu_out_f64(y_u), gpu_out_f64(y_f))
    print(f"[report] unfused vs fused {name} {fmt} M={M}: rel_fro={rf:.3e}", flush=True)


@pytest.mark.parametrize("name,fmt,M", [("tiny", "block", 1), ("tiny", "mx", 1), ("d2048", "block", 1),
                                        ("d2048", "block", 16), ("d4096", "mx", 1), ("d4096", "mx", 16),
                                        ("d4096", "mx", 64), ("d4096", "mx", 128), ("d2560", "block", 64)])
def test_unfused_pipeline_parity(name, fmt, M):
    d = dev()
    note(f"unfused pipeline {name} {fmt} M={M}")
    _unfused(name, fmt, M, d)
