"""fp64 reference computations (CPU oracle; test infrastructure only).

* Scaled GEMM: Y = deq(Xq) deq(Wq)^T -- the block-scaled (1x128 activation
  groups x 128x128 weight tiles) and MX (1x32 UE8M0 on both operands) FP8
  GEMMs of fish.audio blog, section "Qué hay en código abierto", evaluated as
  the plain definition in float64 after bit-exact quantization.
* SwiGLU MLP: y = (silu(x Wg^T) * (x Wu^T)) Wd^T -- the "activation, gate
  multiplication, down projection" layer of Fish Audio X post, section
  "Custom kernels for the shapes TTS actually uses"; SiLU is applied to the
  gate branch (Shazeer 2020, "GLU Variants Improve Transformer", Swish with
  beta = 1).  The product is re-quantized as the down GEMM's activation
  (fish.audio blog, section "Resultados de benchmark del kernel": the SwiGLU
  prologue is fused into the down-GEMM activation quantization).  It is
  rounded to fp32 before that quantization, as the GPU path quantizes from
  fp32.
* Decode stack: pre-RMSNorm residual SwiGLU blocks (RMSNorm as in Zhang &
  Sennrich 2019, "Root Mean Square Layer Normalization", unit gain,
  eps = 1e-6, no final norm), then a bf16 output head with fp32-or-better
  logits and a per-row argmax with the lowest index winning ties.  The
  correctness gate this stands in for is greedy decode matching token for
  token (X post, section "FP8 only works if quality survives").  bf16
  roundings happen exactly where the GPU path rounds: the normalised input
  of each block, each block output and the head input; the residual stream
  is held in fp32 (each residual add rounds to fp32), as on the GPU.

Every matmul here is numpy's float64 matmul on dequantized (exact) values.
"""

import numpy as np

from .fp8 import to_bf16
from .quant import quantize_act, quantize_weight, dequantize_act, dequantize_weight

RMS_EPS = 1e-6


class QWeight:
    """An oracle-quantized weight: codes [N, K] uint8, scales (logical)."""

    def __init__(self, w, fmt):
        w = np.asarray(w, dtype=np.float64)
        self.fmt = fmt
        self.N, self.K = w.shape
        self.codes, self.scales = quantize_weight(w, fmt)

    def deq(self):
        return dequantize_weight(self.codes, self.scales, self.fmt)


def gemm_quantized(xq, xs, wq, ws, fmt):
    """Y[m, n] = sum_k deq(xq)[m, k] * deq(wq)[n, k] in float64."""
    return dequantize_act(xq, xs, fmt) @ dequantize_weight(wq, ws, fmt).T


def scaled_gemm(x, qw):
    """Quantize x [M, K] per row (qw.fmt), then the fp64 scaled GEMM."""
    xq, xs = quantize_act(x, qw.fmt)
    return dequantize_act(xq, xs, qw.fmt) @ qw.deq().T


def silu(g):
    """g * sigmoid(g) = g / (1 + exp(-g)), float64."""
    g = np.asarray(g, dtype=np.float64)
    with np.errstate(over="ignore"):
        return g / (1.0 + np.exp(-g))


def swiglu_mlp(x, qg, qu, qd, return_all=False):
    """The quantized SwiGLU MLP on x [M, d] (float64 holding bf16 values).

    1. (xq, sx) = Q(x) per row along d;
    2. g = deq(xq) deq(Wg)^T, u = deq(xq) deq(Wu)^T   (float64);
    3. a = silu(g) * u;
    4. a32 = fl32(a);
    5. (aq, sa) = Q(a32) per row along ffn;
    6. y = deq(aq) deq(Wd)^T   (float64).
    """
    fmt = qg.fmt
    assert qu.fmt == fmt and qd.fmt == fmt
    xq, sx = quantize_act(x, fmt)
    xd = dequantize_act(xq, sx, fmt)
    g = xd @ qg.deq().T
    u = xd @ qu.deq().T
    a = silu(g) * u
    a32 = a.astype(np.float32).astype(np.float64)
    aq, sa = quantize_act(a32, fmt)
    y = dequantize_act(aq, sa, fmt) @ qd.deq().T
    if return_all:
        return dict(y=y, xq=xq, sx=sx, g=g, u=u, a=a, a32=a32, aq=aq, sa=sa)
    return y


def swiglu_mlp_unquantized(x, wg, wu, wd):
    """The same MLP without any quantization (float64 throughout)."""
    x = np.asarray(x, dtype=np.float64)
    g = x @ np.asarray(wg, dtype=np.float64).T
    u = x @ np.asarray(wu, dtype=np.float64).T
    return (silu(g) * u) @ np.asarray(wd, dtype=np.float64).T


def rmsnorm(h, eps=RMS_EPS):
    """h / sqrt(mean(h^2) + eps) per row, unit gain, float64."""
    h = np.asarray(h, dtype=np.float64)
    return h / np.sqrt(np.mean(h * h, axis=1, keepdims=True) + eps)


def block_output(h, qg, qu, qd, eps=RMS_EPS):
    """The residual branch of one pre-norm block: bf16(MLP(bf16(RMSNorm(h))))."""
    xl = to_bf16(rmsnorm(h, eps))
    return to_bf16(swiglu_mlp(xl, qg, qu, qd))


def residual_add(h, y):
    """h + y rounded to fp32 (the residual stream is fp32)."""
    return (np.asarray(h, dtype=np.float64) + np.asarray(y, dtype=np.float64)).astype(np.float32).astype(np.float64)


def stack_layer(h, qg, qu, qd, eps=RMS_EPS):
    """One pre-norm residual block: fl32(h + bf16(MLP(bf16(RMSNorm(h)))))."""
    return residual_add(h, block_output(h, qg, qu, qd, eps))


def head_logits(h, w_head):
    """logits = bf16(h) W_head^T in float64 (W_head holds bf16 values)."""
    return to_bf16(h) @ np.asarray(w_head, dtype=np.float64).T


def argmax_rows(logits):
    """Per-row argmax; np.argmax returns the lowest index among ties."""
    return np.argmax(np.asarray(logits), axis=1)


# --------------------------------------------------------------------------
# error metrics
# --------------------------------------------------------------------------

def rel_fro(y, ref):
    """||y - ref||_F / ||ref||_F."""
    y = np.asarray(y, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.linalg.norm(y - ref) / np.linalg.norm(ref))


def max_abs_ratio(y, ref):
    """max|y - ref| / max|ref|."""
    y = np.asarray(y, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.max(np.abs(y - ref)) / np.max(np.abs(ref)))


# Acceptance bar for GEMM / MLP outputs against this oracle.
REL_FRO_TOL = 5e-3
MAX_ABS_TOL = 2e-2
