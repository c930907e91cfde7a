"""GPU parity of scaled_gemm and the fused SwiGLU MLP against the oracle at
sizes the oracle finishes in seconds (several tiles, ragged row counts), plus
edge cases and the permuted-scale negative test."""

import numpy as np
import pytest
import torch

import swiglu_decode_amd as sgd
import synth
from oracle import ref
from synth import bf16_to_f64
from tests.gpu_util import assert_close, dev, gpu_out_f64, note, oracle_weight

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("fmt", ["block", "mx"])
@pytest.mark.parametrize("M", [1, 2, 16, 17, 40, 64, 100, 128])
@pytest.mark.parametrize("N,K", [(256, 512), (384, 1152)])
def test_scaled_gemm_parity(fmt, M, N, K):
    d = dev()
    note(f"scaled_gemm {fmt} M={M} N={N} K={K}")
    x = synth.random_bf16((M, K), 11 + M, 1.0)
    w = synth.random_bf16((N, K), 12 + N, 0.02)
    pw = sgd.quantize_pack_weight(w.to(d), fmt)
    y = sgd.scaled_gemm(x.to(d), pw)
    torch.cuda.synchronize()
    y_ref = ref.scaled_gemm(bf16_to_f64(x), oracle_weight(w, fmt))
    assert_close(gpu_out_f64(y), y_ref, f"gemm {fmt} M={M} {N}x{K}")


_big = {}


def _big_weight(N, K, fmt, d):
    """One full-size weight at a time (bounded host memory): bf16, the
    oracle's quantized copy and the packed GPU copy."""
    key = (N, K, fmt)
    if key not in _big:
        _big.clear()
        w = synth.random_bf16((N, K), 900 + N // 128 + K // 128, 0.02)
        _big[key] = (w, oracle_weight(w, fmt), sgd.quantize_pack_weight(w.to(d), fmt))
    return _big[key]


@pytest.mark.parametrize("fmt", ["block", "mx"])
@pytest.mark.parametrize("N,K", [(12288, 4096), (4096, 12288)])
@pytest.mark.parametrize("M", [1, 16, 64, 128])
def test_scaled_gemm_full_size(fmt, N, K, M):
    """The plain GEMM at the MLP's own shapes (gate/up: 12288 x 4096, down:
    4096 x 12288): the second-GEMM bands are split over several workgroups and
    combined (split-K) at every row-tile count."""
    d = dev()
    note(f"scaled_gemm full size {fmt} M={M} N={N} K={K}")
    w, qw, pw = _big_weight(N, K, fmt, d)
    x = synth.random_bf16((M, K), 21 + M, 1.0)
    ws = sgd.Workspace(d, sgd.gemm_workspace_bytes(fmt, M, N, K))
    y = sgd.scaled_gemm(x.to(d), pw, workspace=ws)
    y2 = sgd.scaled_gemm(x.to(d), pw, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(y, y2), "a second call on the same workspace changed the result"
    y_ref = ref.scaled_gemm(bf16_to_f64(x), qw)
    assert_close(gpu_out_f64(y), y_ref, f"gemm {fmt} M={M} {N}x{K}")


@pytest.mark.parametrize("fmt", ["block", "mx"])
@pytest.mark.parametrize("M", [1, 5, 16, 33, 48, 64, 100, 128])
@pytest.mark.parametrize("d_,F", [(256, 768), (512, 1536), (640, 1152)])
def test_fused_mlp_parity(fmt, M, d_, F):
    d = dev()
    note(f"fused_mlp {fmt} M={M} d={d_} F={F}")
    wl = synth.Workload("t", d_, F, (M,), (fmt,), 2000 + d_ + F)
    inp = synth.mlp_inputs(wl, M)
    pws = [sgd.quantize_pack_weight(inp[k].to(d), fmt) for k in ("wg", "wu", "wd")]
    y = sgd.fused_swiglu_mlp(inp["x"].to(d), *pws)
    torch.cuda.synchronize()
    q = [oracle_weight(inp[k], fmt) for k in ("wg", "wu", "wd")]
    y_ref = ref.swiglu_mlp(bf16_to_f64(inp["x"]), *q)
    assert_close(gpu_out_f64(y), y_ref, f"mlp {fmt} M={M} d={d_} F={F}")


@pytest.mark.parametrize("fmt", ["block", "mx"])
def test_repeated_calls_and_shrinking_m_share_a_workspace(fmt):
    # the control block must be left ready: back-to-back calls, then a smaller M
    d = dev()
    note(f"repeat {fmt}")
    wl = synth.Workload("t", 512, 1536, (64,), (fmt,), 3001)
    inp = synth.mlp_inputs(wl, 64)
    pws = [sgd.quantize_pack_weight(inp[k].to(d), fmt) for k in ("wg", "wu", "wd")]
    ws = sgd.Workspace(d, sgd.mlp_workspace_bytes(fmt, 64, 512, 1536))
    x = inp["x"].to(d)
    ys = [sgd.fused_swiglu_mlp(x, *pws, workspace=ws).clone() for _ in range(5)]
    torch.cuda.synchronize()
    for y in ys[1:]:
        assert torch.equal(y, ys[0])
    y3 = sgd.fused_swiglu_mlp(x[:3].contiguous(), *pws, workspace=ws)
    torch.cuda.synchronize()
    q = [oracle_weight(inp[k], fmt) for k in ("wg", "wu", "wd")]
    assert_close(gpu_out_f64(ys[0]), ref.swiglu_mlp(bf16_to_f64(inp["x"]), *q), "repeat M=64")
    assert_close(gpu_out_f64(y3), ref.swiglu_mlp(bf16_to_f64(inp["x"][:3]), *q), "shrink M=3")


@pytest.mark.parametrize("fmt", ["block", "mx"])
def test_zero_and_outlier_inputs(fmt):
    d = dev()
    note(f"edge inputs {fmt}")
    wl = synth.Workload("t", 512, 1024, (8,), (fmt,), 3002)
    inp = synth.mlp_inputs(wl, 8)
    x = inp["x"].float()
    x[0] = 0.0                  # an all-zero row
    x[1, :128] = 0.0            # an all-zero group
    x[2, 7] = 3000.0            # an outlier channel
    x[3] *= 1e-6                # small-magnitude row (results stay in the fp32 normal range)
    x = x.to(torch.bfloat16)
    pws = [sgd.quantize_pack_weight(inp[k].to(d), fmt) for k in ("wg", "wu", "wd")]
    y = sgd.fused_swiglu_mlp(x.to(d), *pws)
    torch.cuda.synchronize()
    q = [oracle_weight(inp[k], fmt) for k in ("wg", "wu", "wd")]
    yr = ref.swiglu_mlp(bf16_to_f64(x), *q)
    yg = gpu_out_f64(y)
    assert np.all(yg[0] == 0.0)
    for r in range(1, 8):
        if np.any(yr[r] != 0):
            assert_close(yg[r:r + 1], yr[r:r + 1], f"edge row {r}")


@pytest.mark.parametrize("fmt", ["block", "mx"])
def test_permuted_scales_are_caught(fmt):
    # The failure class the pages describe: a scale buffer in the wrong layout
    # gives full-speed wrong results.  Feed the kernel a scale buffer whose
    # entries are permuted and check the parity gate fails by a wide margin.
    d = dev()
    note(f"negative scales {fmt}")
    wl = synth.Workload("t", 512, 1536, (4,), (fmt,), 3003)
    inp = synth.mlp_inputs(wl, 4)
    # give the down weight strongly varying per-tile magnitudes
    wd = inp["wd"].float()
    mult = torch.exp2(torch.arange(wd.shape[1] // 128).float() % 5 - 2)
    wd = (wd * mult.repeat_interleave(128)[None, :]).to(torch.bfloat16)
    pws = [sgd.quantize_pack_weight(t.to(d), fmt) for t in (inp["wg"], inp["wu"], wd)]
    good = sgd.fused_swiglu_mlp(inp["x"].to(d), *pws).clone()
    s = pws[2].scales
    if fmt == "block":
        sv = s.view(torch.float32).view(512 // 128, 1536 // 128)
        bad_s = sv.flip(1).contiguous().view(torch.uint8).view(-1)
    else:
        bad_s = s.view(-1, 4).flip(1).contiguous().view(-1)
    bad_w = sgd.PackedWeight(pws[2].fmt, pws[2].N, pws[2].K, pws[2].codes, bad_s)
    bad = sgd.fused_swiglu_mlp(inp["x"].to(d), pws[0], pws[1], bad_w)
    torch.cuda.synchronize()
    q = [oracle_weight(t, fmt) for t in (inp["wg"], inp["wu"], wd)]
    yr = ref.swiglu_mlp(bf16_to_f64(inp["x"]), *q)
    assert_close(gpu_out_f64(good), yr, "negative-test control")
    err = ref.rel_fro(gpu_out_f64(bad), yr)
    print(f"[parity] permuted scales rel_fro={err:.3f}")
    assert err > 0.1


# Word of the control block that counts completed launches (flags are raised
# with the current launch's number, so they need no clearing between calls).
LAUNCH_COUNT_WORD = 64


@pytest.mark.parametrize("fmt,M", [("mx", 4), ("block", 64), ("mx", 128)])
def test_launch_number_wrap(fmt, M):
    # preset the launch count just below 2**32 - 1: the calls then use launch
    # numbers 0xFFFFFFFE, 0xFFFFFFFF (which clears every flag on exit), 1, 2;
    # each must equal the first call on a fresh workspace, bit for bit
    d = dev()
    note(f"launch-number wrap {fmt} M={M}")
    wl = synth.Workload("t", 1024, 3072, (M,), (fmt,), 3004)
    inp = synth.mlp_inputs(wl, M)
    pws = [sgd.quantize_pack_weight(inp[k].to(d), fmt) for k in ("wg", "wu", "wd")]
    x = inp["x"].to(d)
    ws0 = sgd.Workspace(d, sgd.mlp_workspace_bytes(fmt, M, 1024, 3072))
    y0 = sgd.fused_swiglu_mlp(x, *pws, workspace=ws0).clone()
    ws = sgd.Workspace(d, sgd.mlp_workspace_bytes(fmt, M, 1024, 3072))
    ws.tensor[4 * LAUNCH_COUNT_WORD:4 * LAUNCH_COUNT_WORD + 4].copy_(
        torch.tensor([0xFD, 0xFF, 0xFF, 0xFF], dtype=torch.uint8))
    ys = [sgd.fused_swiglu_mlp(x, *pws, workspace=ws).clone() for _ in range(4)]
    torch.cuda.synchronize()
    count = int(ws.tensor[4 * LAUNCH_COUNT_WORD:4 * LAUNCH_COUNT_WORD + 4].cpu().view(torch.int32)[0])
    assert count == 2, count
    for i, y in enumerate(ys):
        assert torch.equal(y, y0), f"call {i} after the preset differs"
    q = [oracle_weight(inp[k], fmt) for k in ("wg", "wu", "wd")]
    assert_close(gpu_out_f64(y0), ref.swiglu_mlp(bf16_to_f64(inp["x"]), *q), f"wrap {fmt} M={M}")
