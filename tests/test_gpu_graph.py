"""The fused MLP and the scaled GEMM captured in a HIP graph: 100 replays,
with eager work and synchronisations between them, each equal to the eager
result bit for bit (the kernels leave the workspace's control block ready
for the next launch, with counters zero and flags holding the launch number,
and record no memset)."""

import pytest
import torch

import swiglu_decode_amd as sgd
import synth
from tests.gpu_util import dev, note

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("fmt,M", [("block", 4), ("mx", 16), ("mx", 64), ("block", 128)])
def test_graph_replay_matches_eager(fmt, M):
    d = dev()
    note(f"graph replay {fmt} M={M}")
    wl = synth.Workload("g", 2048, 6144, (M,), (fmt,), 4001)
    inp = synth.mlp_inputs(wl, M)
    pws = [sgd.quantize_pack_weight(inp[k].to(d), fmt) for k in ("wg", "wu", "wd")]
    x = inp["x"].to(d)
    ws = sgd.Workspace(d, max(sgd.mlp_workspace_bytes(fmt, M, 2048, 6144),
                              sgd.gemm_workspace_bytes(fmt, M, 6144, 2048)))
    y = torch.empty((M, 2048), dtype=torch.bfloat16, device=d)
    g = torch.empty((M, 6144), dtype=torch.bfloat16, device=d)
    st = torch.cuda.Stream()
    with torch.cuda.stream(st):
        sgd.fused_swiglu_mlp(x, *pws, out=y, workspace=ws)
        sgd.scaled_gemm(x, pws[0], out=g, workspace=ws)
        st.synchronize()
        y_eager, g_eager = y.clone(), g.clone()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=st):
            sgd.fused_swiglu_mlp(x, *pws, out=y, workspace=ws)
            sgd.scaled_gemm(x, pws[0], out=g, workspace=ws)
        for r in range(100):
            y.zero_()
            g.zero_()
            st.synchronize()
            graph.replay()
            st.synchronize()
            assert torch.equal(y, y_eager), f"replay {r}: MLP output differs from the eager call"
            assert torch.equal(g, g_eager), f"replay {r}: GEMM output differs from the eager call"
            # eager work between replays on the same workspace
            sgd.fused_swiglu_mlp(x, *pws, out=y, workspace=ws)
            st.synchronize()
            assert torch.equal(y, y_eager)
