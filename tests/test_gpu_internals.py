"""GPU parity of the fused kernel's own intermediates, read back from its
workspace (sgd_mlp_workspace_layout):

* Q(x): the kernel's in-kernel quantizer (clamp to +-448, then the hardware
  E4M3 conversion; IEEE division for the block scale) must give the same
  codes and scales as the oracle's integer encoder, bit for bit, on every
  finite bf16 value and on values planted at scale edges.
* Q(a): the re-quantization of a = silu(g) * u.  The kernel's fp32 product a
  is read back and quantized by the oracle; the kernel's Q(a) must equal it
  bit for bit (both sides take the fp8 decision on the same fp32 value).  a
  itself is compared with the oracle's fp64 product to fp32 accuracy.

These reach the split-K combine of shared gate/up bands at one and two row
tiles (d=2560, ffn=9728 at M <= 32) as well as the staged path (M > 32)."""

import numpy as np
import pytest
import torch

import swiglu_decode_amd as sgd
import synth
from oracle import fp8, quant, ref
from synth import bf16_to_f64
from tests.gpu_util import dev, note, oracle_weight

pytestmark = pytest.mark.gpu


def _mpad(M):
    return 16 if M <= 16 else 32 if M <= 32 else 64 if M <= 64 else 128


def mtile_codes(buf, M, K):
    """[M, K] codes from the m-tile layout (16-column segments, Mt rows each)."""
    out = np.empty((M, K), dtype=np.uint8)
    for t in range(0, M, 16):
        Mt = min(16, M - t)
        seg = buf[t * K:t * K + Mt * K].reshape(K // 16, Mt, 16)
        out[t:t + Mt] = seg.transpose(1, 0, 2).reshape(Mt, K)
    return out


def mtile_scales(buf, M, K, fmt):
    """Logical scales (block fp32 [M, K/128]; mx E8M0 [M, K/32]) from the
    workspace layout (block: fp32 [K/128][Mpad]; mx: per m-tile and k-tile
    one dword of four E8M0 bytes per row)."""
    if fmt == "block":
        s = buf[:(K // 128) * _mpad(M) * 4].view(np.float32).reshape(K // 128, _mpad(M))
        return np.ascontiguousarray(s.T[:M])
    out = np.empty((M, K // 32), dtype=np.uint8)
    KT = K // 128
    for t in range(0, M, 16):
        Mt = min(16, M - t)
        base = t * (K // 32)
        blk = buf[base:base + KT * Mt * 4].reshape(KT, Mt, 4)
        out[t:t + Mt] = blk.transpose(1, 0, 2).reshape(Mt, K // 32)
    return out


def _run(x_cpu, pws, fmt, M, d, ffn, ws):
    dv = pws[0].device
    y = sgd.fused_swiglu_mlp(x_cpu.to(dv), *pws, workspace=ws)
    torch.cuda.synchronize()
    assert ws.status() == 0
    off = sgd.mlp_workspace_layout(fmt, M, d, ffn)
    buf = ws.tensor.cpu().numpy()
    return y, off, buf


def _assert_scales_equal(got, want, fmt, what):
    if fmt == "block":
        assert np.array_equal(got.view(np.uint32), want.astype(np.float32).view(np.uint32)), what
    else:
        assert np.array_equal(got, want), what


def _all_bf16_x(M, K, seed):
    bits = np.arange(65536, dtype=np.uint16)
    vals = fp8.bf16_bits_to_f64(bits)
    vals = vals[np.isfinite(vals)]
    buf = np.zeros(M * K)
    buf[:vals.size] = vals
    np.random.default_rng(seed).shuffle(buf)
    x = torch.from_numpy(buf.reshape(M, K).astype(np.float32)).to(torch.bfloat16)
    assert np.array_equal(bf16_to_f64(x), buf.reshape(M, K))
    return x


def _special_x(M, K, seed):
    x = synth.random_bf16((M, K), seed, 1.0).float()
    x[0, :128] = 0.0                        # an all-zero group
    x[1, 0:32] = -0.0                       # signed zeros
    x[2, 40] = 3.0e38                       # huge amax
    x[3, 7] = 2.0 ** -130                   # bf16 subnormal, alone in its block
    x[3, 0:7] = 0.0
    x[3, 8:32] = 0.0
    x[4, 0:4] = torch.tensor([448.0, 464.0, 480.0, -0.5])  # e4m3 edges at scale 1
    return x.to(torch.bfloat16)


def _weights(d, ffn, fmt, seed):
    wg = synth.random_bf16((ffn, d), seed, 0.02)
    wu = synth.random_bf16((ffn, d), seed + 1, 0.02)
    wd = synth.random_bf16((d, ffn), seed + 2, 0.02)
    return wg, wu, wd


@pytest.mark.parametrize("fmt", ["block", "mx"])
@pytest.mark.parametrize("M,d,xkind", [(64, 1024, "all_bf16"), (20, 4096, "special"), (128, 512, "special")])
def test_kernel_x_quantizer_bit_exact(fmt, M, d, xkind):
    """Q(x) as the kernel stores it for M > 32 (or when x does not fit in LDS)."""
    dv = dev()
    ffn = 1024
    note(f"in-kernel Q(x) {fmt} M={M} d={d} x={xkind}")
    x = _all_bf16_x(M, d, 11) if xkind == "all_bf16" else _special_x(M, d, 12 + M)
    pws = [sgd.quantize_pack_weight(w.to(dv), fmt) for w in _weights(d, ffn, fmt, 300)]
    ws = sgd.Workspace(dv, sgd.mlp_workspace_bytes(fmt, M, d, ffn))
    _, off, buf = _run(x, pws, fmt, M, d, ffn, ws)
    c_ref, s_ref = quant.quantize_act(bf16_to_f64(x), fmt)
    codes = mtile_codes(buf[off["xq"]:], M, d)
    bad = np.argwhere(codes != c_ref)
    assert bad.size == 0, [(int(r), int(c), int(codes[r, c]), int(c_ref[r, c])) for r, c in bad[:8]]
    _assert_scales_equal(mtile_scales(buf[off["xs"]:], M, d, fmt), s_ref, fmt, "Q(x) scales")


REQ_CASES = [(1, 1024, 2048), (16, 1024, 2048), (17, 1024, 2048), (33, 1024, 2048), (48, 1024, 2048),
             (64, 1024, 2048), (100, 1024, 2048), (128, 1024, 2048),
             # shared gate/up bands (split-K combine) at one and two row tiles
             (1, 2560, 9728), (16, 2560, 9728), (32, 2560, 9728)]


@pytest.mark.parametrize("fmt", ["block", "mx"])
@pytest.mark.parametrize("M,d,ffn", REQ_CASES)
def test_kernel_requant_bit_exact(fmt, M, d, ffn):
    dv = dev()
    note(f"in-kernel a and Q(a) {fmt} M={M} d={d} ffn={ffn}")
    x = synth.random_bf16((M, d), 40 + M, 1.0)
    w = _weights(d, ffn, fmt, 500 + d)
    pws = [sgd.quantize_pack_weight(t.to(dv), fmt) for t in w]
    ws = sgd.Workspace(dv, sgd.mlp_workspace_bytes(fmt, M, d, ffn))
    # (a is kept in the workspace for this check: above 32 rows the kernel
    # re-quantizes from registers and stores a only when asked to)
    prev = sgd.set_keep_intermediates(True)
    try:
        _, off, buf = _run(x, pws, fmt, M, d, ffn, ws)
    finally:
        sgd.set_keep_intermediates(prev)
    a_gpu = buf[off["a"]:off["a"] + M * ffn * 4].view(np.float32).reshape(M, ffn).astype(np.float64)
    # the product itself, against the oracle's fp64 one (fp32 accumulation)
    q = [oracle_weight(t, fmt) for t in w]
    o = ref.swiglu_mlp(bf16_to_f64(x), *q, return_all=True)
    rf = ref.rel_fro(a_gpu, o["a"])
    print(f"[parity] a = silu(g)*u {fmt} M={M} d={d} ffn={ffn}: rel_fro={rf:.3e}", flush=True)
    # gate/up on the bf16 matrix instruction after an exact widening has
    # fp32-accurate sums; the staged schedule (64-row tiles in MX, 128-row
    # tiles in both formats) runs it on the scaled fp8 one, whose sums keep
    # about 13 bits below the largest product of each group of 8 (~1e-4 per
    # group, ~2e-5 over the whole sum)
    f8 = M > 64 or (M > 32 and fmt == "mx")
    tol = 1e-4 if f8 else 1e-5
    assert rf <= tol, rf
    # Q(a) from the kernel's own a, bit for bit
    c_ref, s_ref = quant.quantize_act(a_gpu, fmt)
    codes = mtile_codes(buf[off["aq"]:], M, ffn)
    bad = np.argwhere(codes != c_ref)
    assert bad.size == 0, [(int(r), int(c), int(codes[r, c]), int(c_ref[r, c])) for r, c in bad[:8]]
    _assert_scales_equal(mtile_scales(buf[off["as_"]:], M, ffn, fmt), s_ref, fmt, "Q(a) scales")
