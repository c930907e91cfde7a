"""GPU parity of the large-M (prefill) path: Q(x) in 16-row tiles, the
LDS-tiled scaled fp8 GEMM, and the prefill SwiGLU MLP built from them,
against the oracle (and against the decode path where both apply)."""

import numpy as np
import pytest
import torch

import swiglu_decode_amd as sgd
import synth
from oracle import quant, ref
from synth import bf16_to_f64
from tests.gpu_util import assert_close, dev, gpu_out_f64, note, oracle_weight

pytestmark = pytest.mark.gpu

CTRL = 256 * 1024  # the large path leaves the workspace's control block alone


def _a256(v):
    return (v + 255) // 256 * 256


def _tiles_codes(buf, Mpad, K):
    """[Mpad, K] codes from the full-tile layout (16-column segments of 16 rows)."""
    return buf[:Mpad * K].reshape(Mpad // 16, K // 16, 16, 16).transpose(0, 2, 1, 3).reshape(Mpad, K)


def _tiles_scales(buf, Mpad, K, fmt):
    if fmt == "block":
        return buf[:(K // 128) * Mpad * 4].view(np.float32).reshape(K // 128, Mpad).T
    return buf[:Mpad * (K // 32)].reshape(Mpad // 16, K // 128, 16, 4).transpose(0, 2, 1, 3).reshape(Mpad, K // 32)


@pytest.mark.parametrize("fmt", ["block", "mx"])
@pytest.mark.parametrize("M,K", [(1, 512), (300, 1024)])
def test_act_tiles_bit_exact(fmt, M, K):
    """Q(x) of the large path (read back from the workspace) equals the
    oracle's quantizer byte for byte; padded rows hold zero codes (block:
    zero scales)."""
    d = dev()
    note(f"large-path Q(x) tiles {fmt} M={M} K={K}")
    x = synth.random_bf16((M, K), 900 + M, 3.0)
    w = sgd.quantize_pack_weight(synth.random_bf16((128, K), 901, 0.02).to(d), fmt)
    ws = sgd.Workspace(d, sgd.lib().sgd_gemm_large_workspace_bytes(sgd.fmt_code(fmt), M, 128, K))
    sgd.scaled_gemm_large(x.to(d), w, workspace=ws)
    torch.cuda.synchronize()
    buf = ws.tensor.cpu().numpy()[CTRL:]
    Mpad = (M + 15) // 16 * 16
    codes = _tiles_codes(buf, Mpad, K)
    scales = _tiles_scales(buf[_a256(Mpad * K):], Mpad, K, fmt)
    c_ref, s_ref = quant.quantize_act(bf16_to_f64(x), fmt)
    np.testing.assert_array_equal(codes[:M], c_ref)
    np.testing.assert_array_equal(scales[:M], s_ref)
    assert np.all(codes[M:] == 0)
    if fmt == "block":
        assert np.all(scales[M:] == 0)


@pytest.mark.parametrize("fmt", ["block", "mx"])
@pytest.mark.parametrize("M,N,K", [(1, 256, 512), (64, 384, 640), (129, 512, 1024), (300, 1152, 768),
                                   (1000, 1024, 2048)])
def test_gemm_large_parity(fmt, M, N, K):
    d = dev()
    note(f"large GEMM {fmt} M={M} N={N} K={K}")
    x = synth.random_bf16((M, K), 910 + M, 1.0)
    w = synth.random_bf16((N, K), 911 + N, 0.02)
    pw = sgd.quantize_pack_weight(w.to(d), fmt)
    y = sgd.scaled_gemm_large(x.to(d), pw)
    torch.cuda.synchronize()
    assert_close(gpu_out_f64(y), ref.scaled_gemm(bf16_to_f64(x), oracle_weight(w, fmt)), f"large gemm {fmt} M={M}")
    if M <= 128:  # the decode path's result, up to the order of the fp32 sums
        y2 = sgd.scaled_gemm(x.to(d), pw)
        torch.cuda.synchronize()
        assert ref.rel_fro(gpu_out_f64(y), gpu_out_f64(y2)) <= 2e-3


@pytest.mark.parametrize("fmt", ["block", "mx"])
def test_gemm_large_square_4096_sampled(fmt):
    """4096^3 (the pages' square benchmark family), checked on two whole rows
    and 256 sampled entries computed by the oracle one by one."""
    d = dev()
    S = 4096
    note(f"large GEMM {fmt} {S}^3 sampled")
    x = synth.random_bf16((S, S), 920, 1.0)
    w = synth.random_bf16((S, S), 921, 0.02)
    pw = sgd.quantize_pack_weight(w.to(d), fmt)
    y = sgd.scaled_gemm_large(x.to(d), pw).float().cpu().numpy().astype(np.float64)
    rng = np.random.default_rng(922)
    rows = np.concatenate([[0, S - 1], rng.integers(0, S, 256)])
    cols = rng.integers(0, S, 256)
    qw = oracle_weight(w, fmt)
    wd = qw.deq()
    xq, xs = quant.quantize_act(bf16_to_f64(x[rows]), fmt)
    xr = quant.dequantize_act(xq, xs, fmt)
    full = xr[:2] @ wd.T
    assert_close(y[rows[:2]], full, f"large gemm {fmt} {S}^3 rows 0 and {S - 1}")
    got = y[rows[2:], cols]
    want = np.einsum("ik,ik->i", xr[2:], wd[cols])
    assert_close(got, want, f"large gemm {fmt} {S}^3 sampled entries")


@pytest.mark.parametrize("name,fmt,M", [("tiny", "block", 5), ("d2048", "block", 200), ("d2560", "mx", 77)])
def test_mlp_prefill_parity(name, fmt, M):
    d = dev()
    note(f"prefill MLP {name} {fmt} M={M}")
    wl = synth.WORKLOADS[name]
    inp = synth.mlp_inputs(wl, 1)
    rng = np.random.default_rng(930 + M)
    x = torch.from_numpy(rng.standard_normal((M, wl.d)).astype(np.float32)).to(torch.bfloat16)
    pg, pu, pd = [sgd.quantize_pack_weight(inp[k].to(d), fmt) for k in ("wg", "wu", "wd")]
    y = sgd.swiglu_mlp_prefill(x.to(d), sgd.stack_packed(pg, pu), pd)
    torch.cuda.synchronize()
    q = [oracle_weight(inp[k], fmt) for k in ("wg", "wu", "wd")]
    assert_close(gpu_out_f64(y), ref.swiglu_mlp(bf16_to_f64(x), *q), f"prefill MLP {name} {fmt} M={M}")
    if M <= 128:
        yf = sgd.fused_swiglu_mlp(x.to(d), pg, pu, pd)
        torch.cuda.synchronize()
        rf = ref.rel_fro(gpu_out_f64(y), gpu_out_f64(yf))
        print(f"[report] prefill vs fused {name} {fmt} M={M}: rel_fro={rf:.3e}", flush=True)


@pytest.mark.parametrize("fmt", ["block", "mx"])
def test_mlp_prefill_uneven_ksplit(fmt):
    """d=1024, ffn=4480 (35 k-tiles), M=100: the down projection's 8 blocks
    split K in two ranges of 17 and 18 k-tiles, the second starting inside a
    group of four MX scale k-tiles; the fp32 partials summed by the second
    kernel.  Against the oracle."""
    d = dev()
    note(f"prefill MLP d=1024 ffn=4480 {fmt} M=100 (split K)")
    wl = synth.Workload("ksplit", 1024, 4480, (100,), (fmt,), 1011)
    inp = synth.mlp_inputs(wl)
    M = 100
    x = inp["x"][:M]
    pg, pu, pd = [sgd.quantize_pack_weight(inp[k].to(d), fmt) for k in ("wg", "wu", "wd")]
    y = sgd.swiglu_mlp_prefill(x.to(d), sgd.stack_packed(pg, pu), pd)
    torch.cuda.synchronize()
    q = [oracle_weight(inp[k], fmt) for k in ("wg", "wu", "wd")]
    assert_close(gpu_out_f64(y), ref.swiglu_mlp(bf16_to_f64(x), *q), f"prefill MLP split K {fmt}")


def test_mlp_prefill_d4096_m1024_sampled_rows():
    """d=4096, ffn=12288 MXFP8 at M=1024: 24 sampled rows against the oracle
    (rows of the MLP are independent)."""
    d = dev()
    M = 1024
    note(f"prefill MLP d4096 mx M={M} sampled rows")
    wl = synth.WORKLOADS["d4096"]
    inp = synth.mlp_inputs(wl, 1)
    rng = np.random.default_rng(940)
    x = torch.from_numpy(rng.standard_normal((M, wl.d)).astype(np.float32)).to(torch.bfloat16)
    pg, pu, pd = [sgd.quantize_pack_weight(inp[k].to(d), "mx") for k in ("wg", "wu", "wd")]
    y = sgd.swiglu_mlp_prefill(x.to(d), sgd.stack_packed(pg, pu), pd)
    y2 = sgd.swiglu_mlp_prefill(x.to(d), sgd.stack_packed(pg, pu), pd)
    torch.cuda.synchronize()
    assert torch.equal(y, y2), "the tiled path is not deterministic"
    rows = np.concatenate([[0, M - 1], rng.integers(0, M, 22)])
    q = [oracle_weight(inp[k], "mx") for k in ("wg", "wu", "wd")]
    assert_close(gpu_out_f64(y)[rows], ref.swiglu_mlp(bf16_to_f64(x[rows]), *q), "prefill MLP d4096 M=1024 rows")


@pytest.mark.parametrize("fmt", ["block", "mx"])
def test_gemm_large_max_rows_sampled(fmt):
    """The largest row count (SGD_MAX_M_LARGE = 65536): every output element
    is written (the output starts as NaN) and nonzero rows come back, and 32
    sampled rows, the last ones included, match the oracle."""
    d = dev()
    M, N, K = 65536, 256, 512
    note(f"large GEMM {fmt} M={M} N={N} K={K} sampled rows")
    x = synth.random_bf16((M, K), 950, 1.0)
    w = synth.random_bf16((N, K), 951, 0.02)
    pw = sgd.quantize_pack_weight(w.to(d), fmt)
    y = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device=d)
    sgd.scaled_gemm_large(x.to(d), pw, out=y)
    torch.cuda.synchronize()
    yc = gpu_out_f64(y)
    assert np.all(np.isfinite(yc)) and np.all(np.abs(yc).max(axis=1) > 0)
    rng = np.random.default_rng(952)
    rows = np.concatenate([[0, M - 16, M - 1], rng.integers(0, M, 29)])
    assert_close(yc[rows], ref.scaled_gemm(bf16_to_f64(x[rows]), oracle_weight(w, fmt)),
                 f"large gemm {fmt} M={M} sampled rows")


def test_large_path_keeps_control_block():
    """A large-path call on a workspace shared with the persistent kernels
    leaves their control block as they left it: the fused MLP still works
    (and agrees with itself) after it."""
    d = dev()
    note("large path and fused MLP sharing one workspace")
    wl = synth.WORKLOADS["d2048"]
    inp = synth.mlp_inputs(wl, 16)
    pg, pu, pd = [sgd.quantize_pack_weight(inp[k].to(d), "block") for k in ("wg", "wu", "wd")]
    x = inp["x"][:16].contiguous().to(d)
    ws = sgd.Workspace(d)
    y0 = sgd.fused_swiglu_mlp(x, pg, pu, pd, workspace=ws)
    xl = torch.randn((600, wl.d), device=d).to(torch.bfloat16)
    sgd.swiglu_mlp_prefill(xl, sgd.stack_packed(pg, pu), pd, workspace=ws)
    y1 = sgd.fused_swiglu_mlp(x, pg, pu, pd, workspace=ws)
    torch.cuda.synchronize()
    assert ws.status() == 0
    assert torch.equal(y0, y1)
