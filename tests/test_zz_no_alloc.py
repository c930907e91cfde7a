"""The fused-MLP entry point that allocates nothing
(sgd_fused_swiglu_mlp_noalloc: its workspace is the library's fixed
per-device array) against the workspace entry point on the same inputs: two
calls in a row, the second with fewer rows, each bit-identical to
sgd_fused_swiglu_mlp and within the oracle's tolerance."""

import pytest
import torch

import swiglu_decode_amd as sgd
import synth
from oracle import ref
from synth import bf16_to_f64
from tests.gpu_util import assert_close, dev, gpu_out_f64, note, oracle_weight

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("fmt,d,ffn,M1,M2", [("mx", 1024, 3072, 64, 5), ("block", 2048, 6144, 16, 1)])
def test_noalloc_matches_workspace_entry(fmt, d, ffn, M1, M2):
    dv = dev()
    wl = synth.Workload("noalloc", d, ffn, (M1,), (fmt,), 4100 + d)
    inp = synth.mlp_inputs(wl, M1)
    pws = [sgd.quantize_pack_weight(inp[k].to(dv), fmt) for k in ("wg", "wu", "wd")]
    q = [oracle_weight(inp[k], fmt) for k in ("wg", "wu", "wd")]
    ws = sgd.Workspace(dv, sgd.mlp_workspace_bytes(fmt, M1, d, ffn))
    for M in (M1, M2):
        note(f"no-alloc entry {fmt} d={d} ffn={ffn} M={M}")
        x = inp["x"][:M].contiguous().to(dv)
        y_na = torch.empty((M, d), dtype=torch.bfloat16, device=dv)
        sgd.fused_swiglu_mlp_noalloc(x, *pws, out=y_na)
        y_ws = sgd.fused_swiglu_mlp(x, *pws, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(y_na, y_ws), f"M={M}: the no-alloc entry differs from the workspace entry"
        assert_close(gpu_out_f64(y_na), ref.swiglu_mlp(bf16_to_f64(inp["x"][:M]), *q), f"no-alloc M={M}")
