"""Benchmark: fused FP8 SwiGLU MLP, µs/call and achieved HBM GB/s at M = 1/16/64/128.

Headline workload: SwiGLU MLP with d=4096, ffn=12288, MXFP8 (1x32 UE8M0
scales on both operands), bf16 activations ~ N(0,1), weights N(0, 0.02),
synthetic and seeded.  One step = one fused_swiglu_mlp launch at each M in
{1, 16, 64, 128}; `value` is the step's aggregate algorithmic bytes divided
by its time, in GB/s.

Timing: the packed weights are copied R times (>= 1.1 GB in total, four times
the 256 MB Infinity Cache) and every launch uses the next copy, so weights
are read cold from HBM.  For each M a HIP graph of R launches (one per copy)
is captured and replayed; HIP events on the launch stream bracket each timed
replay.  Algorithmic bytes per launch = fp8 weight codes + weight scales +
bf16 x + bf16 y; intermediates and activation scales are not counted.

Per M the line also carries: the per-call time's p10/p50/p90 over the timed
replays and over >= 200 single eager launches (each bracketed by its own
events), a "warm" figure (every launch on the same weights: cache-resident,
labelled so), and the unfused pipeline (gate/up GEMM into fp32, standalone
SwiGLU + re-quantization, down GEMM from Q(a); intermediates through HBM)
timed the same way, with the fused/unfused ratio.

`roofline` describes the M=16 launch (the >= 70 %-of-peak target case);
`per_config` times the other workloads: d=2048 ffn=6144 128x128-block at
M=1/4/16 (also a target case), d=5120 ffn=13824 at M=64 in both formats,
the 24-block decode step (d=2560 ffn=9728 block, M=64, bf16 head) as one
hipGraph with its per-layer MLP time, and d=256 ffn=768 M=1 (launch-bound,
latency only).  `read_stream_ceiling` is the rate of a plain streaming read
on the same GPU (context).  `cpu_baseline` times the CPU oracle on a bounded
sample on this host, with all cores and single-threaded.  `regression`
compares the M=1/16/64 figures of the headline workload and the d=2048
workload's M=1/4/16 with the frozen ones in bench_frozen.json and flags any
more than 5 % slower (--fail-on-regression turns a flag into exit status 3;
--freeze-from FILE writes the frozen file from an earlier run's line).
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
FROZEN_FILE = os.path.join(ROOT, "bench_frozen.json")
KERNEL_SOURCES = ["swiglu_decode_amd/csrc/stream.hip", "swiglu_decode_amd/csrc/sgd_device.hpp",
                  "swiglu_decode_amd/csrc/sgd_act.hpp"]
REGRESSION_TOL = 0.05


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


def pct(vals, q):
    import numpy as np
    return round(float(np.percentile(np.asarray(vals), q)), 3)


def time_replays(torch, stream, graph, steps, warmup, calls):
    """Replay `graph` warmup times, then `steps` times each bracketed by its
    own pair of events; returns per-call µs of each timed replay."""
    for _ in range(warmup):
        graph.replay()
    stream.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for e0, e1 in ev:
        e0.record(stream)
        graph.replay()
        e1.record(stream)
    stream.synchronize()
    return [e0.elapsed_time(e1) * 1e3 / calls for e0, e1 in ev]


def time_eager(torch, stream, launches, n):
    """n single launches (cycling through `launches`), each bracketed by its
    own events on the stream: per-call device µs."""
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for i, (e0, e1) in enumerate(ev):
        e0.record(stream)
        launches[i % len(launches)]()
        e1.record(stream)
    stream.synchronize()
    return [e0.elapsed_time(e1) * 1e3 for e0, e1 in ev]


def capture(torch, stream, fns):
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for f in fns:
            f()
    return g


class MlpSetup:
    """Seeded inputs, packed weights and R rotation copies (plus the stacked
    gate/up weight of each copy for the unfused pipeline) of one workload."""

    def __init__(self, dev, d, F, fmt, m_max, seed, rotate_bytes, kind="gauss", unfused=True):
        import numpy as np
        import torch
        import swiglu_decode_amd as sgd
        import synth
        self.d, self.F, self.fmt = d, F, fmt
        wl = synth.Workload("bench", d, F, (m_max,), (fmt,), seed, kind=kind)
        self.inp = synth.mlp_inputs(wl, m_max)
        pw0 = [sgd.quantize_pack_weight(self.inp[k].to(dev), fmt) for k in ("wg", "wu", "wd")]
        self.scale_bytes = sum(int(p.scales.numel()) for p in pw0)
        set_bytes = sum(int(p.codes.numel()) + int(p.scales.numel()) for p in pw0)
        self.R = max(2, int(np.ceil(rotate_bytes / set_bytes)))
        self.copies = [pw0] + [[sgd.PackedWeight(p.fmt, p.N, p.K, p.codes.clone(), p.scales.clone()) for p in pw0]
                               for _ in range(self.R - 1)]
        self.stacked = [sgd.stack_packed(c[0], c[1]) for c in self.copies] if unfused else None
        self.x_all = self.inp["x"].to(dev)
        self.ws = sgd.Workspace(dev, sgd.mlp_workspace_bytes(fmt, m_max, d, F))
        self.ws_gemm = sgd.Workspace(dev, max(sgd.gemm_workspace_bytes(fmt, m_max, 2 * F, d),
                                              sgd.gemm_workspace_bytes(fmt, m_max, d, F)))
        torch.cuda.synchronize()

    def bytes(self, M):
        return algorithmic_bytes(M, self.d, self.F, self.scale_bytes)


def bench_m(torch, sgd, st, dev, stream, M, steps, warmup, eager_n, unfused=True, warm=True):
    """Fused (and unfused) timing of one M on one MlpSetup."""
    x = st.x_all[:M].contiguous()
    y = torch.empty((M, st.d), dtype=torch.bfloat16, device=dev)
    with torch.cuda.stream(stream):
        sgd.fused_swiglu_mlp(x, *st.copies[0], out=y, workspace=st.ws)
        stream.synchronize()
        g = capture(torch, stream, [lambda r=r: sgd.fused_swiglu_mlp(x, *st.copies[r], out=y, workspace=st.ws)
                                    for r in range(st.R)])
        reps = time_replays(torch, stream, g, steps, warmup, st.R)
        y_out = y.float().cpu().numpy()
        eager = time_eager(torch, stream, [lambda r=r: sgd.fused_swiglu_mlp(x, *st.copies[r], out=y, workspace=st.ws)
                                           for r in range(st.R)], eager_n) if eager_n else None
        del g
        res = {}
        if warm:
            gw = capture(torch, stream, [lambda: sgd.fused_swiglu_mlp(x, *st.copies[0], out=y, workspace=st.ws)]
                         * st.R)
            res["warm_us_per_call"] = round(sum(time_replays(torch, stream, gw, max(3, steps // 4), 2, st.R))
                                            / max(3, steps // 4), 3)
            del gw
        if unfused:
            gu = torch.empty((M, 2 * st.F), dtype=torch.float32, device=dev)
            aq = torch.empty(M * st.F, dtype=torch.uint8, device=dev)
            sc = torch.empty(sgd.lib().sgd_act_scales_bytes(sgd.fmt_code(st.fmt), M, st.F), dtype=torch.uint8,
                             device=dev)
            yu = torch.empty((M, st.d), dtype=torch.bfloat16, device=dev)
            run_u = [lambda r=r: sgd.unfused_swiglu_mlp(x, st.stacked[r], st.copies[r][2], out=yu,
                                                         workspace=st.ws_gemm, buffers=(gu, aq, sc))
                     for r in range(st.R)]
            run_u[0]()
            stream.synchronize()
            gg = capture(torch, stream, run_u)
            ureps = time_replays(torch, stream, gg, max(5, steps // 2), 2, st.R)
            del gg
            res["unfused_us_per_call"] = round(sum(ureps) / len(ureps), 3)
    us = sum(reps) / len(reps)
    b = st.bytes(M)
    out = dict(us_per_call=round(us, 3), bytes=b, gbs=round(b / us / 1e3, 1),
               pct_of_peak=round(100.0 * b / us / 1e3 / HBM_PEAK_GBS, 1),
               replay_p10_p50_p90=[pct(reps, 10), pct(reps, 50), pct(reps, 90)], timed_calls=len(reps) * st.R)
    if eager:
        out.update(eager_p10_p50_p90=[pct(eager, 10), pct(eager, 50), pct(eager, 90)], eager_calls=len(eager))
    out.update(res)
    if "unfused_us_per_call" in out:
        out["unfused_over_fused"] = round(out["unfused_us_per_call"] / out["us_per_call"], 3)
    return out, y_out


def bench_stack(torch, sgd, dev, steps, warmup):
    """The decode step of the 24-block stack: h = f32(x); 24 blocks, each ONE
    launch (sgd_fused_swiglu_block: RMSNorm prologue, fused MLP, residual
    epilogue, h alternating between two fp32 buffers); then the bf16 head and
    the argmax of every row.  All 24 packed layers stay resident (1.8 GB, far
    beyond the Infinity Cache, so each step reads them cold); the step is
    captured once as a hipGraph and replayed, timed with HIP events on its
    stream.  The 24 block launches alone are timed the same way (per-block
    figure), and so is the same step built from separate launches (RMSNorm,
    fused MLP, and the residual add fused with the next RMSNorm), for
    comparison.  Algorithmic bytes per step = per block (fp8 weights + scales
    + fp32 h in + fp32 h out) + bf16 head + f32 logits."""
    import synth
    eps = 1e-6  # RMSNorm epsilon of the stack
    wl = synth.WORKLOADS["stack"]
    M, d, F = wl.ms[0], wl.d, wl.ffn
    layers = [[sgd.quantize_pack_weight(w.to(dev), "block") for w in synth.stack_layer_weights(wl, layer)]
              for layer in range(wl.layers)]
    head = synth.stack_head(wl).to(dev)
    x = synth.stack_x(wl, M).to(dev)
    ha = torch.empty((M, d), dtype=torch.float32, device=dev)
    hb = torch.empty((M, d), dtype=torch.float32, device=dev)
    xb = torch.empty((M, d), dtype=torch.bfloat16, device=dev)
    y = torch.empty((M, d), dtype=torch.bfloat16, device=dev)
    lg = torch.empty((M, wl.vocab), dtype=torch.float32, device=dev)
    tok = torch.empty((M,), dtype=torch.int32, device=dev)
    ws = sgd.Workspace(dev, sgd.mlp_workspace_bytes("block", M, d, F))
    layer_bytes = sum(int(p.codes.numel()) + int(p.scales.numel()) for p in layers[0]) + 2 * M * d * 4
    step_bytes = wl.layers * layer_bytes + int(head.numel()) * 2 + M * wl.vocab * 4

    def blocks():
        cur, nxt = ha, hb
        for pws in layers:
            sgd.fused_swiglu_block(cur, *pws, eps=eps, out=nxt, workspace=ws)
            cur, nxt = nxt, cur
        return cur

    def step():
        sgd.bf16_to_f32(x, out=ha)
        h = blocks()
        sgd.head_logits(h, head, out=lg)
        sgd.argmax_rows(lg, out=tok)

    def step_separate():
        sgd.bf16_to_f32(x, out=ha)
        sgd.rmsnorm_bf16(ha, eps, out=xb)
        for i, pws in enumerate(layers):
            sgd.fused_swiglu_mlp(xb, *pws, out=y, workspace=ws)
            if i + 1 < len(layers):
                sgd.residual_rmsnorm_bf16(ha, y, eps, out=xb)
            else:
                sgd.residual_add(ha, y)
        sgd.head_logits(ha, head, out=lg)
        sgd.argmax_rows(lg, out=tok)

    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        step()
        stream.synchronize()
        tok_eager = tok.clone()
        lg_eager = lg.clone()
        g = capture(torch, stream, [step])
        reps = time_replays(torch, stream, g, steps, warmup, 1)
        graph_equal = bool(torch.equal(tok, tok_eager)) and bool(torch.equal(lg, lg_eager))
        del g
        gl = capture(torch, stream, [blocks])
        lreps = time_replays(torch, stream, gl, steps, 2, wl.layers)
        del gl
        step_separate()
        stream.synchronize()
        separate_equal = bool(torch.equal(lg, lg_eager))
        gs = capture(torch, stream, [step_separate])
        sreps = time_replays(torch, stream, gs, max(5, steps // 2), 2, 1)
        del gs
    us = sum(reps) / len(reps)
    lus = sum(lreps) / len(lreps)
    sus = sum(sreps) / len(sreps)
    out = dict(workload=f"{wl.layers} x (RMSNorm, fused SwiGLU MLP d={d} ffn={F} 128x128 block fp8, residual add: "
                        f"one launch per block) + bf16 head {wl.vocab}x{d} + argmax, M={M}, one hipGraph",
               us_per_step=round(us, 2), step_p10_p50_p90=[pct(reps, 10), pct(reps, 50), pct(reps, 90)],
               us_per_block=round(us / wl.layers, 2), algorithmic_bytes_per_step=step_bytes,
               gbs=round(step_bytes / us / 1e3, 1), pct_of_peak=round(100.0 * step_bytes / us / 1e3 / HBM_PEAK_GBS, 1),
               fused_block_us_per_layer=round(lus, 2),
               fused_block_layer_pct_of_peak=round(100.0 * layer_bytes / lus / 1e3 / HBM_PEAK_GBS, 1),
               separate_launches_us_per_step=round(sus, 2),
               separate_launches_logits_equal=separate_equal,
               graph_tokens_equal_eager=graph_equal)
    del layers
    torch.cuda.empty_cache()
    return out


FP8_PEAK_TFLOPS = 5000.0  # MI355X dense fp8 matrix peak


def bench_large(torch, sgd, dev):
    """The large-M (prefill) path, MFMA-bound: square scaled GEMMs S^3
    (x [S, S] bf16 quantized per row, packed [S, S] weight; 2 S^3 flop per
    call) and the prefill SwiGLU MLP at d=4096, ffn=12288 (6 M d ffn flop).
    Each call includes its x quantization.  Seeded synthetic inputs (x
    N(0,1), weights N(0,0.02)); R calls captured back to back in one hipGraph
    (R up to 16, about 2 ms of work), timed with HIP events on its stream."""

    def timed(fn, n):
        # R back-to-back calls captured in one graph (no host launch gaps
        # between them), replayed n times; per-call time = replay / R
        s = torch.cuda.Stream()
        with torch.cuda.stream(s):
            fn()
            s.synchronize()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(s)
            fn()
            e1.record(s)
            e1.synchronize()
            R = max(1, min(16, int(2000.0 / max(e0.elapsed_time(e1) * 1e3, 1.0))))
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=s):
                for _ in range(R):
                    fn()
            g.replay()
            s.synchronize()
            times = []
            for _ in range(n):
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record(s)
                g.replay()
                e1.record(s)
                e1.synchronize()
                times.append(e0.elapsed_time(e1) * 1e3 / R)
        del g
        return times

    def entry(flop, times):
        us = sum(times) / len(times)
        tf = flop / us / 1e6
        return dict(us_per_call=round(us, 2), p10_p50_p90=[pct(times, 10), pct(times, 50), pct(times, 90)],
                    tflops=round(tf, 1), roofline=dict(bound="mfma", achieved=round(tf, 1), peak=FP8_PEAK_TFLOPS,
                                                       unit="TFLOP/s", frac=round(tf / FP8_PEAK_TFLOPS, 4)))

    g = torch.Generator(device=dev)
    g.manual_seed(1007)
    out = {}
    for fmt, sizes in (("mx", (1024, 2048, 4096, 8192, 16384)), ("block", (4096, 8192))):
        for S in sizes:
            x = torch.randn((S, S), device=dev, generator=g).to(torch.bfloat16)
            w = sgd.quantize_pack_weight((torch.randn((S, S), device=dev, generator=g) * 0.02).to(torch.bfloat16), fmt)
            y = torch.empty((S, S), dtype=torch.bfloat16, device=dev)
            ws = sgd.Workspace(dev, sgd.lib().sgd_gemm_large_workspace_bytes(sgd.fmt_code(fmt), S, S, S))
            t = timed(lambda: sgd.scaled_gemm_large(x, w, out=y, workspace=ws), 5 if S >= 8192 else 20)
            out[f"gemm_{fmt}_{S}^3"] = entry(2.0 * S ** 3, t)
            del x, w, y, ws
            torch.cuda.empty_cache()
    d, F = 4096, 12288
    for fmt, ms in (("mx", (512, 1024, 4096)), ("block", (4096,))):
        pw = [sgd.quantize_pack_weight((torch.randn(s, device=dev, generator=g) * 0.02).to(torch.bfloat16), fmt)
              for s in ((F, d), (F, d), (d, F))]
        gu = sgd.stack_packed(pw[0], pw[1])
        for M in ms:
            x = torch.randn((M, d), device=dev, generator=g).to(torch.bfloat16)
            y = torch.empty((M, d), dtype=torch.bfloat16, device=dev)
            ws = sgd.Workspace(dev, sgd.lib().sgd_mlp_prefill_workspace_bytes(sgd.fmt_code(fmt), M, d, F))
            t = timed(lambda: sgd.swiglu_mlp_prefill(x, gu, pw[2], out=y, workspace=ws), 10)
            out[f"prefill_mlp_d{d}_ffn{F}_{fmt}_M{M}"] = entry(6.0 * M * d * F, t)
            del x, y, ws
        del pw, gu
        torch.cuda.empty_cache()
    return out


def bench_attention(torch, sgd, dev, steps):
    """Paged decode attention over an MXFP8 K/V cache, HBM-bound: batch 64,
    32 query heads over 8 KV heads of head_dim 128 (the decode stack's
    d = 2560 model), sequence lengths uniform on [256, 4096], pages shuffled.
    Bytes per call = the K and V codes and scales of every sequence's tokens
    + bf16 q and out.  Timed with HIP events over graph replays of R calls
    over R cache copies (so each call reads its cache cold)."""
    import numpy as np
    import synth
    B, Hq, Hkv, lo, hi = 64, 32, 8, 256, 4096
    inp = synth.attention_inputs(B, Hq, Hkv, lo, hi, 2400)
    n_pages = inp["n_pages"]
    lens = inp["lens"]
    slots = np.concatenate([inp["pages"][b, np.arange(T) // 16] * 16 + np.arange(T) % 16
                            for b, T in enumerate(lens)]).astype(np.int32)
    cache_bytes = sgd.lib().sgd_kv_cache_bytes(n_pages, Hkv)
    R = max(2, int(np.ceil(1.1e9 / (2 * cache_bytes))))
    st = torch.from_numpy(slots).to(dev)
    k0 = sgd.kv_cache_alloc(n_pages, Hkv, dev)
    v0 = sgd.kv_cache_alloc(n_pages, Hkv, dev)
    off = 0
    for b, T in enumerate(lens):
        sl = st[off:off + T]
        sgd.kv_cache_write("k", inp["k"][b, :T].contiguous().to(dev), sl, k0, n_pages)
        sgd.kv_cache_write("v", inp["v"][b, :T].contiguous().to(dev), sl, v0, n_pages)
        off += T
    kcs, vcs = [k0] + [k0.clone() for _ in range(R - 1)], [v0] + [v0.clone() for _ in range(R - 1)]
    q = inp["q"].to(dev)
    pages = torch.from_numpy(inp["pages"]).to(dev)
    lt = torch.from_numpy(lens).to(dev)
    out = torch.empty((B, Hq, 128), dtype=torch.bfloat16, device=dev)
    ws = sgd.Workspace(dev)
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        sgd.paged_decode_attention(q, k0, v0, n_pages, pages, lt, Hkv, out=out, workspace=ws)
        stream.synchronize()
        g = capture(torch, stream, [lambda r=r: sgd.paged_decode_attention(q, kcs[r], vcs[r], n_pages, pages, lt,
                                                                             Hkv, out=out, workspace=ws)
                                    for r in range(R)])
        reps = time_replays(torch, stream, g, steps, 3, R)
        del g
    us = sum(reps) / len(reps)
    tokens = int(lens.sum())
    nbytes = tokens * Hkv * 2 * (128 + 4) + 2 * B * Hq * 128 * 2
    del kcs, vcs, k0, v0
    torch.cuda.empty_cache()
    return dict(workload=f"paged decode attention, MXFP8 K/V cache (16-slot pages), B={B}, Hq={Hq}, Hkv={Hkv}, "
                         f"head_dim 128, lengths uniform {lo}..{hi} (mean {tokens / B:.0f})",
                us_per_call=round(us, 2), p10_p50_p90=[pct(reps, 10), pct(reps, 50), pct(reps, 90)],
                algorithmic_bytes=nbytes, gbs=round(nbytes / us / 1e3, 1),
                roofline=dict(bound="hbm", achieved=round(nbytes / us / 1e3, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                              frac=round(nbytes / us / 1e3 / HBM_PEAK_GBS, 4)),
                cache_copies_rotated=R)


def cpu_baseline(inp, ms, fmt, y_out, budget_s=10.0):
    """Time the CPU oracle (as it stands) on a bounded sample: passes of one
    MLP call at M=1 and one at M=16 on the headline workload, repeated until
    about `budget_s` of wall time have passed (at most 12 passes), weights
    quantized beforehand (the analogue of the offline pack, untimed); then
    the M=1 call single-threaded (BLAS limited to one thread) for about as
    long.  Returns the baseline in the bench's unit (algorithmic GB/s) and the
    GPU-vs-oracle parity of those calls."""
    import numpy as np
    from threadpoolctl import threadpool_info, threadpool_limits
    from oracle import ref
    from synth import bf16_to_f64
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    q = [ref.QWeight(bf16_to_f64(inp[k]), fmt) for k in ("wg", "wu", "wd")]
    x = bf16_to_f64(inp["x"])
    d = x.shape[1]
    F = q[0].N
    scale_bytes = sum(int(np.asarray(w.scales).nbytes) for w in q)
    sample = [m for m in (1, 16) if m in ms] or [ms[0]]

    def run(sample, budget):
        t_tot, b_tot, passes, ys = 0.0, 0, 0, {}
        while passes < 12 and (passes == 0 or t_tot < budget):
            for m in sample:
                t0 = time.perf_counter()
                ys[m] = ref.swiglu_mlp(x[:m], *q)
                t_tot += time.perf_counter() - t0
                b_tot += algorithmic_bytes(m, d, F, scale_bytes)
            passes += 1
        return t_tot, b_tot, passes, ys

    t_all, b_all, p_all, ys = run(sample, budget_s)
    parity = {str(m): dict(rel_fro=float(f"{ref.rel_fro(y_out[m], ys[m]):.3e}"),
                           max_abs_ratio=float(f"{ref.max_abs_ratio(y_out[m], ys[m]):.3e}")) for m in sample}
    with threadpool_limits(limits=1):
        t_one, b_one, p_one, _ = run(sample[:1], budget_s)
    cpu = dict(value=round(b_all / t_all / 1e9, 4), unit="GB/s", cores=threads, kind="oracle",
               sample=f"{p_all} pass(es) of one oracle MLP call at each M in {sample} on the headline workload "
                      f"(x quantization, fp64 dequantize + matmuls, SwiGLU, re-quantization), weights "
                      f"pre-quantized; {t_all:.1f} s with {threads} BLAS threads on {os.cpu_count()} host CPUs",
               single_thread=dict(value=round(b_one / t_one / 1e9, 4), unit="GB/s", cores=1,
                                  sample=f"{p_one} pass(es) at M={sample[0]}, {t_one:.1f} s"),
               host_cpus=os.cpu_count())
    return cpu, parity


def regression(per_m, d2048):
    """Figures more than 5 % slower than the frozen ones (the pages'
    performance gate: decode throughput within 5 % of frozen baselines at
    batch 1, 16 and 64)."""
    if not os.path.exists(FROZEN_FILE):
        return dict(baseline_file=None, slower_than_5pct=[])
    frozen = json.load(open(FROZEN_FILE))
    now = {f"d4096_mx_M{m}": per_m[str(m)]["us_per_call"] for m in (1, 16, 64) if str(m) in per_m}
    if d2048:
        now.update({f"d2048_block_M{m}": d2048[str(m)]["us_per_call"] for m in (1, 4, 16) if str(m) in d2048})
    slower = []
    for k, v in now.items():
        f = frozen.get("us_per_call", {}).get(k)
        if f and v > f * (1 + REGRESSION_TOL):
            slower.append(dict(case=k, us_per_call=v, frozen=f, ratio=round(v / f, 3)))
    return dict(baseline_file=os.path.basename(FROZEN_FILE), frozen_from=frozen.get("source"), tol=REGRESSION_TOL,
                compared=sorted(now), slower_than_5pct=slower)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=25)  # 25 graph replays of 8 launches: 200 timed calls at d=4096
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--ms", default="1,16,64,128")
    ap.add_argument("--fmt", default="mx")
    ap.add_argument("--d", type=int, default=4096)
    ap.add_argument("--ffn", type=int, default=12288)
    ap.add_argument("--rotate-bytes", type=float, default=1.1e9)
    ap.add_argument("--eager-calls", type=int, default=200)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-read-ceiling", action="store_true",
                    help="skip the plain streaming-read measurement (profiling runs of the fused kernel)")
    ap.add_argument("--only-main", action="store_true",
                    help="time the headline workload only (no per_config, unfused or warm figures): profiling runs")
    ap.add_argument("--attention", action="store_true",
                    help="only the paged decode attention (MXFP8 K/V cache)")
    ap.add_argument("--large", action="store_true",
                    help="only the large-M path (square scaled GEMMs, prefill MLP)")
    ap.add_argument("--stack", action="store_true",
                    help="only the 24-block decode step (d=2560, ffn=9728, block fp8, M=64, bf16 head)")
    ap.add_argument("--freeze-from", default=None,
                    help="write bench_frozen.json from the JSON line of an earlier run (a file) and exit")
    ap.add_argument("--fail-on-regression", action="store_true")
    ap.add_argument("--copy-calibration", type=float, default=0.0,
                    help="instead of the benchmark, run a plain elementwise copy of this many bytes "
                         "(read once, written once) three times: the reference for HBM byte counters")
    args = ap.parse_args()

    if args.freeze_from:
        line = [ln for ln in open(args.freeze_from) if ln.startswith("{")][-1]
        run = json.loads(line)
        frozen = {"source": os.path.basename(args.freeze_from),
                  "us_per_call": {f"d4096_mx_M{m}": run["per_m"][str(m)]["us_per_call"] for m in (1, 16, 64)}}
        if run.get("per_config"):
            frozen["us_per_call"].update({f"d2048_block_M{m}": v["us_per_call"]
                                          for m, v in run["per_config"]["d2048_ffn6144_block"].items()})
        json.dump(frozen, open(FROZEN_FILE, "w"), indent=1)
        print(json.dumps(frozen))
        return

    if args.gpus != 1:
        print(f"bench.py: the library runs on one GPU; --gpus {args.gpus} is not supported "
              "(the MLP would shard over ffn with one all-reduce of y; see the design notes)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import swiglu_decode_amd as sgd

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
        print(json.dumps(bench_stack(torch, sgd, dev, args.steps, args.warmup)))
        return
    if args.large:
        print(json.dumps(bench_large(torch, sgd, dev)))
        return
    if args.attention:
        print(json.dumps(bench_attention(torch, sgd, dev, args.steps)))
        return

    ms = [int(m) for m in args.ms.split(",")]
    d, F, fmt = args.d, args.ffn, args.fmt
    extra = not args.only_main
    st = MlpSetup(dev, d, F, fmt, max(ms), 1003, args.rotate_bytes, unfused=extra)
    stream = torch.cuda.Stream()
    per_m, y_out = {}, {}
    for m in ms:
        per_m[str(m)], y_out[m] = bench_m(torch, sgd, st, dev, stream, m, args.steps, args.warmup,
                                          args.eager_calls if extra else 0, unfused=extra, warm=extra)
    step_us = sum(per_m[str(m)]["us_per_call"] for m in ms)
    step_bytes = sum(per_m[str(m)]["bytes"] for m in ms)
    value = step_bytes / step_us / 1e3
    inp = st.inp
    R = st.R
    del st
    torch.cuda.empty_cache()

    rm = 16 if 16 in ms else ms[0]
    pr = per_m[str(rm)]
    # counter-measured HBM bytes per launch (when taken with the current kernel
    # sources), expressed like `achieved`: bytes per launch / live duration
    tb = read_traffic() if rm == 16 and d == 4096 and F == 12288 and fmt == "mx" else None
    roof = dict(bound="hbm", achieved=pr["gbs"], peak=HBM_PEAK_GBS, unit="GB/s",
                frac=round(pr["gbs"] / HBM_PEAK_GBS, 4),
                traffic=round(tb / pr["us_per_call"] / 1e3, 1) if tb else None, m=rm,
                us_per_launch=pr["us_per_call"], algorithmic_bytes_per_launch=pr["bytes"],
                traffic_bytes_per_launch=int(tb) if tb else None)

    per_config = None
    if extra:
        per_config = {}
        c2 = MlpSetup(dev, 2048, 6144, "block", 16, 1002, args.rotate_bytes)
        per_config["d2048_ffn6144_block"] = {str(m): bench_m(torch, sgd, c2, dev, stream, m, args.steps,
                                                             args.warmup, args.eager_calls)[0] for m in (1, 4, 16)}
        del c2
        for f4 in ("block", "mx"):
            c4 = MlpSetup(dev, 5120, 13824, f4, 64, 1004, args.rotate_bytes, kind="outlier", unfused=False)
            per_config[f"d5120_ffn13824_{f4}_outlier"] = {"64": bench_m(torch, sgd, c4, dev, stream, 64, args.steps,
                                                                        args.warmup, 0, unfused=False,
                                                                        warm=False)[0]}
            del c4
        c1 = MlpSetup(dev, 256, 768, "block", 1, 1001, 0, unfused=False)
        r1 = bench_m(torch, sgd, c1, dev, stream, 1, args.steps, args.warmup, args.eager_calls, unfused=False,
                     warm=False)[0]
        per_config["d256_ffn768_block_latency"] = {"1": dict(us_per_call=r1["us_per_call"],
                                                             eager_p10_p50_p90=r1["eager_p10_p50_p90"],
                                                             note="launch-bound; weights cache-resident")}
        del c1
        torch.cuda.empty_cache()
        per_config["decode_stack_d2560_ffn9728_m64"] = bench_stack(torch, sgd, dev, args.steps, args.warmup)
        per_config["large_m"] = bench_large(torch, sgd, dev)
        per_config["paged_decode_attention"] = bench_attention(torch, sgd, dev, args.steps)

    ceiling = None if args.no_read_ceiling else read_ceiling(dev)

    cpu, parity = (None, None)
    if not args.no_cpu_baseline:
        cpu, parity = cpu_baseline(inp, ms, fmt, y_out)

    reg = regression(per_m, per_config.get("d2048_ffn6144_block") if per_config else None)
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
        "per_m": per_m,
        "roofline": roof,
        "per_config": per_config,
        "read_stream_ceiling": ceiling,
        "cpu_baseline": cpu,
        "parity": parity,
        "regression": reg,
    }
    print(json.dumps(out))
    if args.fail_on_regression and reg["slower_than_5pct"]:
        sys.exit(3)


if __name__ == "__main__":
    main()
