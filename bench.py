"""Benchmark: fused FP8 SwiGLU MLP, µs/call and achieved HBM GB/s at M = 1/16/64/128.

Workload: SwiGLU MLP with d=4096, ffn=12288, MXFP8 (1x32 UE8M0 scales on both
operands), bf16 activations ~ N(0,1), weights N(0, 0.02), synthetic and seeded.
One step = one fused_swiglu_mlp launch at each M in {1, 16, 64, 128}.

Timing: the packed weights are copied R times (>= 1 GiB in total, four times
the 256 MB Infinity Cache) and every launch uses the next copy, so weights are
read cold from HBM.  For each M a HIP graph of R launches (one per copy) is
captured and replayed; HIP events on the launch stream bracket the timed
replays.  Algorithmic bytes per launch = fp8 weight codes + weight scales +
bf16 x + bf16 y; intermediates and activation scales are not counted.

Output: one JSON line (see the keys below).  `value` is the step's aggregate
algorithmic bytes divided by its time, in GB/s.  `roofline` describes the
M=16 launch (the ≥70 %-of-peak target case); `per_m` lists every M.
`read_stream_ceiling` is the rate of a plain streaming read on the same GPU,
reported as context (the roofline peak stays the nominal 8 TB/s).
`cpu_baseline` times the CPU oracle on a bounded sample on this host; the
same oracle outputs are compared with the GPU outputs (`parity`).
"""

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "fused_mlp_d4096_ffn12288_mx_m16_traffic.txt")
KERNEL_SOURCES = ["swiglu_decode_amd/csrc/stream.hip", "swiglu_decode_amd/csrc/sgd_device.hpp"]


def kernel_hash():
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        h.update(open(os.path.join(ROOT, f), "rb").read())
    return h.hexdigest()[:16]


def read_traffic():
    """Counter-measured HBM bytes per launch of the M=16 kernel, if the file
    was taken with the current kernel sources; else None."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    kv = {}
    for line in open(TRAFFIC_FILE):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("kernel_source_sha256_16") != kernel_hash():
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def read_ceiling(dev, nbytes=4 << 30, reps=10):
    """Attainable HBM read rate on this GPU, for context: the library's plain
    streaming-read kernel over `nbytes` of device memory, timed with HIP
    events on the launch stream."""
    import torch
    import swiglu_decode_amd as sgd
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        t = torch.empty(nbytes, dtype=torch.uint8, device=dev)
        sink = torch.empty((1,), dtype=torch.int32, device=dev)
        for _ in range(2):
            sgd.read_stream(t, sink)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            sgd.read_stream(t, sink)
        e1.record(stream)
    e1.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / reps
    del t
    torch.cuda.empty_cache()
    return dict(gbs=round(nbytes / us / 1e3, 1), kernel=f"sgd_read_stream over {nbytes >> 20} MiB",
                pct_of_peak=round(100.0 * nbytes / us / 1e3 / HBM_PEAK_GBS, 1))


def algorithmic_bytes(M, d, F, scale_bytes):
    return 3 * d * F + scale_bytes + 2 * M * d * 2


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--ms", default="1,16,64,128")
    ap.add_argument("--fmt", default="mx")
    ap.add_argument("--d", type=int, default=4096)
    ap.add_argument("--ffn", type=int, default=12288)
    ap.add_argument("--rotate-bytes", type=float, default=1.1e9)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-read-ceiling", action="store_true",
                    help="skip the plain streaming-read measurement (profiling runs of the fused kernel)")
    ap.add_argument("--stack", action="store_true",
                    help="instead of the single-MLP benchmark, time the whole decode step of the 24-block "
                         "stack (d=2560, ffn=9728, 128x128 block fp8, M=64, bf16 head 4096x2560) as one hipGraph")
    ap.add_argument("--copy-calibration", type=float, default=0.0,
                    help="instead of the benchmark, run a plain elementwise copy of this many bytes "
                         "(read once, written once) three times: the reference for HBM byte counters")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU; --gpus {args.gpus} is not supported "
              "(the MLP would shard over ffn with one all-reduce of y; see the design notes)",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.copy_calibration > 0:
        n = int(args.copy_calibration) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_read": 4 * n, "bytes_written": 4 * n, "launches": 3}))
        return

    if args.stack:
        bench_stack(args, dev)
        return

    import swiglu_decode_amd as sgd
    import synth
    ms = [int(m) for m in args.ms.split(",")]
    d, F, fmt = args.d, args.ffn, args.fmt
    wl = synth.Workload("bench", d, F, tuple(ms), (fmt,), 1003)
    inp = synth.mlp_inputs(wl, max(ms))
    x_all = inp["x"].to(dev)
    pw0 = [sgd.quantize_pack_weight(inp[k].to(dev), fmt) for k in ("wg", "wu", "wd")]
    scale_bytes = sum(int(p.scales.numel()) for p in pw0)
    set_bytes = sum(int(p.codes.numel()) + int(p.scales.numel()) for p in pw0)
    R = max(2, int(np.ceil(args.rotate_bytes / set_bytes)))
    copies = [pw0] + [[sgd.PackedWeight(p.fmt, p.N, p.K, p.codes.clone(), p.scales.clone()) for p in pw0]
                      for _ in range(R - 1)]
    ws = sgd.Workspace(dev, sgd.mlp_workspace_bytes(fmt, max(ms), d, F))
    xs = {m: x_all[:m].contiguous() for m in ms}
    ys = {m: torch.empty((m, d), dtype=torch.bfloat16, device=dev) for m in ms}
    torch.cuda.synchronize()

    stream = torch.cuda.Stream()
    graphs = {}
    with torch.cuda.stream(stream):
        for m in ms:  # eager warm-up on the capture stream (first-call host setup)
            sgd.fused_swiglu_mlp(xs[m], *copies[0], out=ys[m], workspace=ws)
        stream.synchronize()
        for m in ms:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=stream):
                for r in range(R):
                    sgd.fused_swiglu_mlp(xs[m], *copies[r], out=ys[m], workspace=ws)
            graphs[m] = g
    torch.cuda.synchronize()

    per_m = {}
    with torch.cuda.stream(stream):
        for m in ms:
            for _ in range(args.warmup):
                graphs[m].replay()
            stream.synchronize()
            t0 = torch.cuda.Event(enable_timing=True)
            t1 = torch.cuda.Event(enable_timing=True)
            t0.record(stream)
            for _ in range(args.steps):
                graphs[m].replay()
            t1.record(stream)
            t1.synchronize()
            us = t0.elapsed_time(t1) * 1e3 / (args.steps * R)
            b = algorithmic_bytes(m, d, F, scale_bytes)
            per_m[m] = dict(us_per_call=round(us, 3), bytes=b, gbs=round(b / us / 1e3, 1),
                            pct_of_peak=round(100.0 * b / us / 1e3 / HBM_PEAK_GBS, 1))
    torch.cuda.synchronize()

    step_us = sum(per_m[m]["us_per_call"] for m in ms)
    step_bytes = sum(per_m[m]["bytes"] for m in ms)
    value = step_bytes / step_us / 1e3

    # outputs of the last replay, for the parity pairing below
    y_out = {m: ys[m].float().cpu().numpy() for m in ms}

    rm = 16 if 16 in ms else ms[0]
    # counter-measured HBM bytes per launch (when taken with the current kernel
    # sources), expressed like `achieved`: bytes per launch / live duration
    tb = read_traffic() if rm == 16 and d == 4096 and F == 12288 and fmt == "mx" else None
    traffic = round(tb / per_m[rm]["us_per_call"] / 1e3, 1) if tb else None
    roof = dict(bound="hbm", achieved=per_m[rm]["gbs"], peak=HBM_PEAK_GBS, unit="GB/s",
                frac=round(per_m[rm]["gbs"] / HBM_PEAK_GBS, 4),
                traffic=traffic, m=rm, us_per_launch=per_m[rm]["us_per_call"],
                algorithmic_bytes_per_launch=per_m[rm]["bytes"],
                traffic_bytes_per_launch=int(tb) if tb else None)

    ceiling = None if args.no_read_ceiling else read_ceiling(dev)

    cpu = None
    parity = None
    if not args.no_cpu_baseline:
        cpu, parity = cpu_baseline(inp, ms, fmt, y_out, step_bytes)

    out = {
        "metric": "fused FP8 SwiGLU µs/call + achieved HBM GB/s (% of peak) at M=1/16/64/128",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_us / 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8_e4m3",
        "data": "synthetic",
        "config": {"workload": f"SwiGLU MLP d={d} ffn={F} {'MXFP8 1x32 UE8M0' if fmt == 'mx' else '128x128 block fp8'}, "
                               f"one fused launch per M in {ms}",
                   "d": d, "ffn": F, "fmt": fmt, "ms": ms, "weight_copies_rotated": R,
                   "parallelism": "single GPU"},
        "per_m": {str(m): per_m[m] for m in ms},
        "roofline": roof,
        "read_stream_ceiling": ceiling,
        "cpu_baseline": cpu,
        "parity": parity,
    }
    print(json.dumps(out))


def bench_stack(args, dev):
    """The decode step of the 24-block stack: h = f32(x); per block
    x_l = bf16(RMSNorm(h)), y_l = fused MLP(x_l), h += y_l (the add and the
    next block's RMSNorm in one launch); then the bf16 head
    and the argmax of every row.  All 24 packed layers stay resident (1.8 GB,
    far beyond the Infinity Cache, so each step reads them cold); the step is
    captured once as a hipGraph and replayed, timed with HIP events on its
    stream.  Algorithmic bytes per step = per block (fp8 weights + scales +
    bf16 x_l + bf16 y_l) + bf16 head + f32 logits."""
    import torch
    import swiglu_decode_amd as sgd
    import synth
    wl = synth.WORKLOADS["stack"]
    M, d, F = wl.ms[0], wl.d, wl.ffn
    layers = []
    for layer in range(wl.layers):
        layers.append([sgd.quantize_pack_weight(w.to(dev), "block") for w in synth.stack_layer_weights(wl, layer)])
    head = synth.stack_head(wl).to(dev)
    x = synth.stack_x(wl, M).to(dev)
    h = torch.empty((M, d), dtype=torch.float32, device=dev)
    xb = torch.empty((M, d), dtype=torch.bfloat16, device=dev)
    y = torch.empty((M, d), dtype=torch.bfloat16, device=dev)
    lg = torch.empty((M, wl.vocab), dtype=torch.float32, device=dev)
    tok = torch.empty((M,), dtype=torch.int32, device=dev)
    ws = sgd.Workspace(dev, sgd.mlp_workspace_bytes("block", M, d, F))
    layer_bytes = sum(int(p.codes.numel()) + int(p.scales.numel()) for p in layers[0]) + 2 * M * d * 2
    step_bytes = wl.layers * layer_bytes + int(head.numel()) * 2 + M * wl.vocab * 4

    def step():
        # (the residual add of a block and the RMSNorm of the next in one launch)
        sgd.bf16_to_f32(x, out=h)
        sgd.rmsnorm_bf16(h, out=xb)
        for i, pws in enumerate(layers):
            sgd.fused_swiglu_mlp(xb, *pws, out=y, workspace=ws)
            if i + 1 < len(layers):
                sgd.residual_rmsnorm_bf16(h, y, out=xb)
            else:
                sgd.residual_add(h, y)
        sgd.head_logits(h, head, out=lg)
        sgd.argmax_rows(lg, out=tok)

    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        step()
        stream.synchronize()
        tok_eager = tok.clone()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            step()
        for _ in range(args.warmup):
            g.replay()
        stream.synchronize()
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        t0.record(stream)
        for _ in range(args.steps):
            g.replay()
        t1.record(stream)
        t1.synchronize()
    us = t0.elapsed_time(t1) * 1e3 / args.steps
    same = bool(torch.equal(tok, tok_eager))
    gbs = step_bytes / us / 1e3
    out = {
        "metric": "decode step of the 24-block fp8 SwiGLU stack: us/step and algorithmic HBM GB/s",
        "value": round(us, 2),
        "unit": "us/step",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(us / 1e3, 5),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8_e4m3",
        "data": "synthetic",
        "config": {"workload": f"{wl.layers} x (RMSNorm, fused SwiGLU MLP d={d} ffn={F} 128x128 block fp8, "
                               f"residual add) + bf16 head {wl.vocab}x{d} + argmax, M={M}, one hipGraph",
                   "layers": wl.layers, "d": d, "ffn": F, "M": M, "vocab": wl.vocab, "fmt": "block",
                   "parallelism": "single GPU"},
        "us_per_block": round(us / wl.layers, 2),
        "algorithmic_bytes_per_step": step_bytes,
        "gbs": round(gbs, 1),
        "pct_of_peak": round(100.0 * gbs / HBM_PEAK_GBS, 1),
        "graph_tokens_equal_eager": same,
    }
    print(json.dumps(out))


def cpu_baseline(inp, ms, fmt, y_out, step_bytes):
    """Time the CPU oracle (as it stands) on a bounded sample: passes of one
    MLP call at M=1 and one at M=16 on the same workload, repeated until about
    10 s of CPU time have passed (at most 12 passes), weights quantized
    beforehand (the analogue of the offline pack, untimed).  Returns the
    baseline in the bench's unit (algorithmic GB/s) and the GPU-vs-oracle
    parity of those calls."""
    import numpy as np
    from oracle import ref
    from synth import bf16_to_f64
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count()
    q = [ref.QWeight(bf16_to_f64(inp[k]), fmt) for k in ("wg", "wu", "wd")]
    x = bf16_to_f64(inp["x"])
    d = x.shape[1]
    F = q[0].N
    scale_bytes = sum(int(np.asarray(w.scales).nbytes) for w in q)
    sample = [m for m in (1, 16) if m in ms] or [ms[0]]
    t_tot, b_tot, passes = 0.0, 0, 0
    parity = {}
    while passes < 12 and (passes == 0 or t_tot < 10.0):
        for m in sample:
            t0 = time.perf_counter()
            y = ref.swiglu_mlp(x[:m], *q)
            t_tot += time.perf_counter() - t0
            b_tot += algorithmic_bytes(m, d, F, scale_bytes)
            if passes == 0:
                parity[str(m)] = dict(rel_fro=float(f"{ref.rel_fro(y_out[m], y):.3e}"),
                                      max_abs_ratio=float(f"{ref.max_abs_ratio(y_out[m], y):.3e}"))
        passes += 1
    cpu = dict(value=round(b_tot / t_tot / 1e9, 4), unit="GB/s", cores=threads, kind="oracle",
               sample=f"{passes} pass(es) of one oracle MLP call at each M in {sample} (x quantization, "
                      f"fp64 dequantize + matmuls, SwiGLU, re-quantization), weights pre-quantized; "
                      f"{t_tot:.1f} s on this host")
    return cpu, parity


if __name__ == "__main__":
    main()
