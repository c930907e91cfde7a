"""GPU tests of the decode block in one launch (sgd_fused_swiglu_block): the
fused SwiGLU MLP with its RMSNorm prologue and residual epilogue,
h_out = fl32(h + bf16(MLP(bf16(RMSNorm(h))))).

It must be bit-identical to the three calls it replaces (RMSNorm to bf16,
the fused MLP, the residual add), whose parts have their own parity tests,
and within the MLP tolerance of the oracle's stack_layer."""

import numpy as np
import pytest
import torch

import swiglu_decode_amd as sgd
import synth
from oracle import ref
from tests.gpu_util import assert_close, dev, note, oracle_weight

pytestmark = pytest.mark.gpu

EPS = ref.RMS_EPS


def _h(M, d, seed):
    """fp32 residual rows of varied scale (RMSNorm sees 0.05..20), the last
    row all zero when M > 2 (RMSNorm gives x = 0, so the block adds nothing)."""
    rng = np.random.default_rng(seed)
    h = rng.standard_normal((M, d)) * np.exp(rng.uniform(np.log(0.05), np.log(20.0), (M, 1)))
    if M > 2:
        h[-1] = 0.0
    return h.astype(np.float32)


def _weights(name, fmt, d):
    wl = synth.WORKLOADS[name]
    inp = synth.mlp_inputs(wl, 1)
    pws = [sgd.quantize_pack_weight(inp[k].to(d), fmt) for k in ("wg", "wu", "wd")]
    return wl, inp, pws


def _three_calls(h, pws, ws):
    xb = sgd.rmsnorm_bf16(h, EPS)
    y = sgd.fused_swiglu_mlp(xb, *pws, workspace=ws)
    hg = h.clone()
    sgd.residual_add(hg, y)
    return hg


@pytest.mark.parametrize("name,fmt,M", [("tiny", "block", 1), ("tiny", "mx", 3), ("d2048", "block", 1),
                                        ("d2048", "block", 16), ("d2560", "block", 33), ("d2560", "block", 64),
                                        ("d2560", "mx", 64), ("d4096", "mx", 1), ("d4096", "mx", 16),
                                        ("d4096", "mx", 128)])
def test_block_bit_identical_to_three_calls(name, fmt, M):
    d = dev()
    note(f"fused block vs rmsnorm + fused MLP + residual add: {name} {fmt} M={M}")
    wl, _, pws = _weights(name, fmt, d)
    h = torch.from_numpy(_h(M, wl.d, 300 + M)).to(d)
    ws = sgd.Workspace(d, sgd.mlp_workspace_bytes(fmt, M, wl.d, wl.ffn))
    want = _three_calls(h, pws, ws)
    got = sgd.fused_swiglu_block(h, *pws, eps=EPS, workspace=ws)
    again = sgd.fused_swiglu_block(h, *pws, eps=EPS, workspace=ws)
    torch.cuda.synchronize()
    assert ws.status() == 0
    assert torch.equal(got, again), "a second call changed the result"
    diff = (got != want).sum().item()
    print(f"[parity] fused block {name} {fmt} M={M}: {diff} of {got.numel()} fp32 values differ from the three calls",
          flush=True)
    assert diff == 0
    if M > 2:  # the zero row: RMSNorm gives 0, the MLP of 0 is 0, h passes through
        assert torch.equal(got[-1], h[-1])


@pytest.mark.parametrize("name,fmt,M", [("tiny", "block", 1), ("d2048", "block", 4), ("d2560", "block", 64),
                                        ("d2560", "mx", 16)])
def test_block_oracle_parity(name, fmt, M):
    """h_out - h against the oracle's block output bf16(MLP(bf16(RMSNorm(h))))
    (both in fp64; the fp32 add costs at most half an fp32 ulp of h_out)."""
    d = dev()
    note(f"fused block vs oracle stack_layer: {name} {fmt} M={M}")
    wl, inp, pws = _weights(name, fmt, d)
    h = _h(M, wl.d, 400 + M)
    got = sgd.fused_swiglu_block(torch.from_numpy(h).to(d), *pws, eps=EPS)
    torch.cuda.synchronize()
    g = got.cpu().numpy().astype(np.float64)
    q = [oracle_weight(inp[k], fmt) for k in ("wg", "wu", "wd")]
    h64 = h.astype(np.float64)
    assert_close(g - h64, ref.block_output(h64, *q, EPS), f"block output {name} {fmt} M={M}")
    # the stored stream is the oracle's fp32 sum of h and the GPU's bf16 output
    np.testing.assert_array_equal(ref.residual_add(h64, g - h64).astype(np.float32), got.cpu().numpy())


def test_block_stack_graph_replays():
    """Three blocks alternating two buffers, captured once as a graph and
    replayed repeatedly with eager work and synchronisation between replays:
    every replay equals the eager run bit for bit."""
    d = dev()
    note("fused block x3 graph replays (d2048 block M=16)")
    wl, _, pws = _weights("d2048", "block", d)
    M = 16
    h0 = torch.from_numpy(_h(M, wl.d, 77)).to(d)
    ha = torch.empty_like(h0)
    hb = torch.empty_like(h0)
    ws = sgd.Workspace(d, sgd.mlp_workspace_bytes("block", M, wl.d, wl.ffn))

    def step():
        sgd.fused_swiglu_block(h0, *pws, eps=EPS, out=ha, workspace=ws)
        sgd.fused_swiglu_block(ha, *pws, eps=EPS, out=hb, workspace=ws)
        sgd.fused_swiglu_block(hb, *pws, eps=EPS, out=ha, workspace=ws)

    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        step()
        s.synchronize()
        want = ha.clone()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            step()
        for i in range(6):
            ha.zero_()
            hb.fill_(float("nan"))
            s.synchronize()
            g.replay()
            s.synchronize()
            assert torch.equal(ha, want), f"replay {i} differs from the eager run"
    assert ws.status() == 0


def test_block_rejects_overlapping_output():
    d = dev()
    note("fused block: output overlapping the input is rejected")
    wl, _, pws = _weights("tiny", "block", d)
    h = torch.zeros((2, wl.d), dtype=torch.float32, device=d)
    with pytest.raises(RuntimeError):
        sgd.fused_swiglu_block(h, *pws, out=h)
