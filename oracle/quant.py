"""Block-128 and MX-32 quantization (CPU oracle; test infrastructure only).

Two formats, both on OCP E4M3 elements:

* ``block`` -- "bsgemm": one fp32 scale per 1x128 activation group (per row,
  along K) and one fp32 scale per 128x128 weight tile.  Fish Audio X post,
  section "Custom kernels for the shapes TTS actually uses" (128x128
  block-scaled FP8); fish.audio blog, sections "Estrategia de cuantización
  FP8" and "Qué hay en código abierto" (1x128 activation x 128x128 weight).
  The scale is s = fl32(amax / 448) and the codes are E4M3(fl32(v / s)),
  with IEEE fp32 division in both places (one amax/448 scale per tile).
* ``mx`` -- "mxfp8": both operands carry one UE8M0 power-of-two scale per
  1x32 block along K.  Same X post section ("1x32 microscaling with OCP
  UE8M0"); fish.audio blog, section "Estrategia de cuantización FP8".  The
  scale follows the OCP MX v1.0 conversion: X = floor(log2(amax)) - 8
  (8 = the E4M3 maximum exponent, 448 = 1.75 * 2^8), clamped to [-127, 127],
  stored as the byte E = X + 127; the codes are E4M3(v * 2^-X), where the
  product is exact and the encoder saturates.

Readings where the pages are silent (listed in the design notes):

* block, amax == 0: s = 1.0 (codes are then all +-0); no epsilon floor.
* block: v / s is a true division (not multiplication by 448/amax).
* mx, amax == 0: E = 0 (X = -127); codes all +-0.
* NaN inputs are outside the contract.

Arrays: bf16 inputs arrive as float64 values (exact).  Activation scales are
laid out [M, K/128] (fp32) or [M, K/32] (uint8 E8M0); weight scales
[N/128, K/128] (fp32) or [N, K/32] (uint8).  Codes are row-major [rows, K].
"""

import numpy as np

from .fp8 import e4m3_encode, e4m3_decode, floor_log2, ue8m0_decode, E4M3_MAX

BLOCK = 128
MX = 32
FMTS = ("block", "mx")


# --------------------------------------------------------------------------
# scale rules (one named function each, so a reading could be swapped)
# --------------------------------------------------------------------------

def block_scale(amax):
    """s = fl32(amax / 448) with IEEE fp32 division; 1.0 where amax == 0."""
    amax32 = np.asarray(amax, dtype=np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        s = amax32 / np.float32(E4M3_MAX)
    return np.where(amax32 == 0, np.float32(1.0), s).astype(np.float32)


def mx_scale_exponent(amax):
    """Unbiased shared exponent X = floor(log2(amax)) - 8, clamped to
    [-127, 127]; X = -127 where amax == 0."""
    amax = np.asarray(amax, dtype=np.float64)
    pos = amax > 0
    X = floor_log2(np.where(pos, amax, 1.0)) - 8
    X = np.where(pos, X, -127)
    return np.clip(X, -127, 127).astype(np.int64)


# --------------------------------------------------------------------------
# quantizers
# --------------------------------------------------------------------------

def _check_k(K, g):
    if K % g:
        raise ValueError(f"K={K} is not a multiple of the group size {g}")


def quantize_act(x, fmt):
    """Per-row quantization of activations x [M, K] (float64 holding bf16 or
    fp32 values) along K.

    Returns (codes uint8 [M, K], scales): block -> fp32 [M, K/128];
    mx -> uint8 E8M0 [M, K/32].  Rows are independent; they are processed a
    few at a time only to bound temporary memory.
    """
    x = np.asarray(x, dtype=np.float64)
    M, K = x.shape
    if fmt not in FMTS:
        raise ValueError(f"unknown format {fmt!r}")
    g = BLOCK if fmt == "block" else MX
    _check_k(K, g)
    codes = np.empty((M, K), dtype=np.uint8)
    scales = np.empty((M, K // g), dtype=np.float32 if fmt == "block" else np.uint8)
    step = max(1, (1 << 16) // K)
    for r in range(0, M, step):
        codes[r:r + step], scales[r:r + step] = _quantize_rows(x[r:r + step], fmt)
    return codes, scales


def _quantize_rows(x, fmt):
    M, K = x.shape
    if fmt == "block":
        xg = x.reshape(M, K // BLOCK, BLOCK)
        s = block_scale(np.abs(xg).max(axis=2))            # [M, K/128] fp32
        q = xg.astype(np.float32) / s[:, :, None]           # IEEE fp32 divide
        return e4m3_encode(q.astype(np.float64)).reshape(M, K), s
    xg = x.reshape(M, K // MX, MX)
    X = mx_scale_exponent(np.abs(xg).max(axis=2))            # [M, K/32]
    q = np.ldexp(xg, (-X)[:, :, None].astype(np.int32))      # exact
    return e4m3_encode(q).reshape(M, K), (X + 127).astype(np.uint8)


def quantize_weight(w, fmt):
    """Quantize a weight matrix w [N, K] (nn.Linear layout: y = x w^T).

    block: one scale per 128x128 tile -> (codes [N, K], fp32 [N/128, K/128]).
    mx:    one scale per 1x32 block along K -> (codes, uint8 [N, K/32]).
    """
    w = np.asarray(w, dtype=np.float64)
    N, K = w.shape
    if fmt == "block":
        _check_k(K, BLOCK)
        if N % BLOCK:
            raise ValueError(f"N={N} is not a multiple of {BLOCK}")
        codes = np.empty((N, K), dtype=np.uint8)
        scales = np.empty((N // BLOCK, K // BLOCK), dtype=np.float32)
        kstep = 16 * BLOCK  # bound temporaries: one band of up to 16 tiles
        for nb in range(N // BLOCK):
            for k0 in range(0, K, kstep):
                band = w[nb * BLOCK:(nb + 1) * BLOCK, k0:k0 + kstep]
                kt = band.shape[1] // BLOCK
                t = band.reshape(BLOCK, kt, BLOCK)
                s = block_scale(np.abs(t).max(axis=(0, 2)))  # [kt]
                q = t.astype(np.float32) / s[None, :, None]
                codes[nb * BLOCK:(nb + 1) * BLOCK, k0:k0 + kstep] = \
                    e4m3_encode(q.astype(np.float64)).reshape(BLOCK, kt * BLOCK)
                scales[nb, k0 // BLOCK:k0 // BLOCK + kt] = s
        return codes, scales
    if fmt == "mx":
        return quantize_act(w, "mx")  # same 1x32-along-K rule per row
    raise ValueError(f"unknown format {fmt!r}")


# --------------------------------------------------------------------------
# dequantizers (exact in float64)
# --------------------------------------------------------------------------

def dequantize_act(codes, scales, fmt):
    """codes [M, K] with per-row group scales -> float64 [M, K]."""
    v = e4m3_decode(codes)
    M, K = v.shape
    if fmt == "block":
        s = np.asarray(scales, dtype=np.float32).astype(np.float64)
        return (v.reshape(M, K // BLOCK, BLOCK) * s[:, :, None]).reshape(M, K)
    if fmt == "mx":
        s = ue8m0_decode(scales)
        return (v.reshape(M, K // MX, MX) * s[:, :, None]).reshape(M, K)
    raise ValueError(f"unknown format {fmt!r}")


def dequantize_weight(codes, scales, fmt):
    """codes [N, K] with weight scales -> float64 [N, K]."""
    v = e4m3_decode(codes)
    N, K = v.shape
    if fmt == "block":
        s = np.asarray(scales, dtype=np.float32).astype(np.float64)
        vt = v.reshape(N // BLOCK, BLOCK, K // BLOCK, BLOCK)
        return (vt * s[:, None, :, None]).reshape(N, K)
    if fmt == "mx":
        return dequantize_act(codes, scales, "mx")
    raise ValueError(f"unknown format {fmt!r}")
