"""The persistent kernels' bounded waits and the binding's ordering of
persistent launches.

* Give-up path: with a wait budget of 1 us set from the host, the waits of
  the fused MLP (Q(x) readiness across workgroups for M > 32, the row
  maxima the bands of a quantization block exchange in the staged schedule,
  Q(a) groups before the second GEMM) outlive it; the kernel must still run to its end
  (the stream synchronises normally), the workspace must report
  SGD_ETIMEOUT, and after a clear a call at the normal budget must be right
  again.  No kernel is made to fault or hang: the condition is forced only
  through the budget the host passes.
* Two streams: calls issued alternately on two streams with the binding's
  per-device default workspace give the same bits as on one stream."""

import pytest
import torch

import swiglu_decode_amd as sgd
import synth
from oracle import ref
from synth import bf16_to_f64
from tests.gpu_util import assert_close, dev, gpu_out_f64, note, oracle_weight

pytestmark = pytest.mark.gpu

ETIMEOUT = -7


def _problem(d, ffn, fmt, M, seed, dv):
    x = synth.random_bf16((M, d), seed, 1.0)
    w = [synth.random_bf16((ffn, d), seed + 1, 0.02), synth.random_bf16((ffn, d), seed + 2, 0.02),
         synth.random_bf16((d, ffn), seed + 3, 0.02)]
    return x, w, [sgd.quantize_pack_weight(t.to(dv), fmt) for t in w]


def test_wait_budget_gives_up_and_every_kernel_exits():
    dv = dev()
    # (64 and 128 rows take the staged schedule: bands exchange their row
    # maxima through flags of their own)
    cases = [(1024, 3072, "mx", 1), (1024, 3072, "block", 64), (2048, 6144, "block", 16), (1024, 3072, "mx", 128)]
    statuses = []
    prev = sgd.set_wait_budget_us(1)
    try:
        for d, ffn, fmt, M in cases:
            note(f"wait budget 1 us: fused MLP {fmt} M={M} d={d} ffn={ffn}")
            x, w, pws = _problem(d, ffn, fmt, M, 70 + M, dv)
            ws = sgd.Workspace(dv, sgd.mlp_workspace_bytes(fmt, M, d, ffn))
            sgd.fused_swiglu_mlp(x.to(dv), *pws, workspace=ws)
            torch.cuda.synchronize()  # the kernel ran to its end
            statuses.append(ws.status())
            print(f"[report] budget 1 us, {fmt} M={M} d={d}: status {statuses[-1]}", flush=True)
    finally:
        sgd.set_wait_budget_us(prev)
    assert all(s in (0, ETIMEOUT) for s in statuses), statuses
    assert ETIMEOUT in statuses, "no wait outlived a 1 us budget"
    # the workspace is usable again after a clear, at the normal budget
    for d, ffn, fmt, M in (cases[0], cases[3]):
        note(f"after give-up: clear and rerun {fmt} M={M}")
        x, w, pws = _problem(d, ffn, fmt, M, 70 + M, dv)
        ws = sgd.Workspace(dv, sgd.mlp_workspace_bytes(fmt, M, d, ffn))
        prev = sgd.set_wait_budget_us(1)
        try:
            sgd.fused_swiglu_mlp(x.to(dv), *pws, workspace=ws)
            torch.cuda.synchronize()
        finally:
            sgd.set_wait_budget_us(prev)
        ws.clear()
        assert ws.status() == 0
        y = sgd.fused_swiglu_mlp(x.to(dv), *pws, workspace=ws)
        torch.cuda.synchronize()
        assert ws.status() == 0
        y_ref = ref.swiglu_mlp(bf16_to_f64(x), *(oracle_weight(t, fmt) for t in w))
        assert_close(gpu_out_f64(y), y_ref, f"after a give-up and a clear, {fmt} M={M}")


def test_two_streams_default_workspace():
    dv = dev()
    d, ffn, fmt = 1024, 3072, "mx"
    note(f"two streams, default workspace, {fmt} d={d} ffn={ffn}")
    xs = {M: _problem(d, ffn, fmt, M, 90, dv) for M in (1, 16, 64)}
    pws = xs[1][2]
    base = {M: sgd.fused_swiglu_mlp(xs[M][0].to(dv), *pws) for M in xs}
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    outs = []
    for i in range(6):
        M = (1, 16, 64)[i % 3]
        with torch.cuda.stream(s1 if i % 2 == 0 else s2):
            outs.append((M, sgd.fused_swiglu_mlp(xs[M][0].to(dv), *pws)))
    torch.cuda.synchronize()
    for M, y in outs:
        assert torch.equal(y, base[M]), M
