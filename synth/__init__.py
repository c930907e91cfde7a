"""Seeded synthetic inputs shared by the GPU path's tests/bench and the oracle.

This module only draws random numbers and rounds them to bf16 (the input
dtype); it holds none of the method's arithmetic.  It imports neither the
oracle nor the GPU package.

Recipe (numpy PCG64 ``default_rng``; samples drawn in float32, scaled in
float32, then rounded to bf16 with round-to-nearest-even by torch's CPU cast):

* weights W_gate, W_up [F, d] and W_down [d, F]: N(0, 0.02), drawn in that
  order from the workload's seed, then x [M_max, d] ~ N(0, 1); a workload
  with several batch sizes uses the first M rows of the same x.
* outlier stress (d=5120, F=13824, M=64): x ~ Student-t(3) with 8 distinct
  randomly chosen channels multiplied by 50 in every row; in each weight
  matrix round(0.001 * F * d) distinct randomly chosen entries are
  multiplied by 20 (drawn after x, in the order gate, up, down).
* decode stack (d=2560, F=9728, 24 layers, M=64): layer l draws its three
  weights from seed 1005 + 100 * l; x from seed 1005 + 9998; the bf16 output
  head [4096, 2560] ~ N(0, 0.02) from seed 1005 + 9999.
* paged decode attention (head_dim 128): sequence lengths uniform on
  [lo, hi] (integers), then q [B, Hq, 128], k and v [B, Tmax, Hkv, 128] all
  N(0, 1), then a random permutation assigning physical 16-slot pages to the
  sequences' logical pages (in sequence order), from one seed.
"""

from dataclasses import dataclass, field
from typing import Tuple

import numpy as np
import torch

WEIGHT_STD = 0.02


@dataclass(frozen=True)
class Workload:
    name: str
    d: int
    ffn: int
    ms: Tuple[int, ...]
    fmts: Tuple[str, ...]
    seed: int
    kind: str = "gauss"          # "gauss" | "outlier" | "stack"
    layers: int = 1
    vocab: int = 0
    note: str = field(default="", compare=False)


WORKLOADS = {
    "tiny": Workload("tiny", 256, 768, (1,), ("block",), 1001,
                     note="single MLP, M=1, d=256, ffn=768, 128x128 block scales"),
    "d2048": Workload("d2048", 2048, 6144, (1, 4, 16), ("block",), 1002,
                      note="MLP d=2048, ffn=6144, 128x128 block scales"),
    "d4096": Workload("d4096", 4096, 12288, (1, 16, 64, 128), ("mx",), 1003,
                      note="MLP d=4096, ffn=12288, MXFP8 1x32 UE8M0"),
    "outlier": Workload("outlier", 5120, 13824, (64,), ("block", "mx"), 1004,
                        kind="outlier",
                        note="outlier stress d=5120, ffn=13824, M=64, both formats"),
    "d2560": Workload("d2560", 2560, 9728, (1, 16, 64), ("block", "mx"), 1006,
                      note="one decode-stack layer's MLP shape (d=2560, ffn=9728) at decode batch sizes"),
    "stack": Workload("stack", 2560, 9728, (64,), ("block",), 1005, kind="stack",
                      layers=24, vocab=4096,
                      note="24 pre-RMSNorm SwiGLU blocks + bf16 head, M=64"),
}


def to_bf16_tensor(a32: np.ndarray) -> torch.Tensor:
    """float32 numpy array -> bf16 CPU tensor (RNE cast)."""
    return torch.from_numpy(np.ascontiguousarray(a32, dtype=np.float32)).to(torch.bfloat16)


def _gauss(rng, shape, std):
    return rng.standard_normal(shape, dtype=np.float32) * np.float32(std)


def mlp_inputs(wl: Workload, m_max: int = None):
    """Return dict(x, wg, wu, wd) of bf16 CPU tensors for a single-MLP
    workload ("gauss" or "outlier")."""
    if m_max is None:
        m_max = max(wl.ms)
    rng = np.random.default_rng(wl.seed)
    d, F = wl.d, wl.ffn
    wg = _gauss(rng, (F, d), WEIGHT_STD)
    wu = _gauss(rng, (F, d), WEIGHT_STD)
    wd = _gauss(rng, (d, F), WEIGHT_STD)
    if wl.kind == "outlier":
        x = rng.standard_t(3, size=(m_max, d)).astype(np.float32)
        ch = rng.choice(d, 8, replace=False)
        x[:, ch] *= np.float32(50.0)
        for w in (wg, wu, wd):
            n = int(round(0.001 * w.size))
            idx = rng.choice(w.size, n, replace=False)
            w.reshape(-1)[idx] *= np.float32(20.0)
    else:
        x = rng.standard_normal((m_max, d), dtype=np.float32)
    return dict(x=to_bf16_tensor(x), wg=to_bf16_tensor(wg),
                wu=to_bf16_tensor(wu), wd=to_bf16_tensor(wd))


def stack_layer_weights(wl: Workload, layer: int):
    """(wg, wu, wd) bf16 CPU tensors of one decode-stack layer."""
    rng = np.random.default_rng(wl.seed + 100 * layer)
    d, F = wl.d, wl.ffn
    wg = _gauss(rng, (F, d), WEIGHT_STD)
    wu = _gauss(rng, (F, d), WEIGHT_STD)
    wd = _gauss(rng, (d, F), WEIGHT_STD)
    return to_bf16_tensor(wg), to_bf16_tensor(wu), to_bf16_tensor(wd)


def stack_x(wl: Workload, m: int = None):
    rng = np.random.default_rng(wl.seed + 9998)
    m = max(wl.ms) if m is None else m
    return to_bf16_tensor(rng.standard_normal((m, wl.d), dtype=np.float32))


def stack_head(wl: Workload):
    rng = np.random.default_rng(wl.seed + 9999)
    return to_bf16_tensor(_gauss(rng, (wl.vocab, wl.d), WEIGHT_STD))


def random_bf16(shape, seed, std=1.0):
    """Generic N(0, std) bf16 CPU tensor (for small parity cases)."""
    rng = np.random.default_rng(seed)
    return to_bf16_tensor(_gauss(rng, shape, std))


def bf16_to_f64(t: torch.Tensor) -> np.ndarray:
    """bf16 tensor -> float64 numpy array (exact)."""
    return t.detach().to("cpu").float().numpy().astype(np.float64)


def attention_inputs(B, Hq, Hkv, lo, hi, seed, extra_pages=0):
    """Seeded decode-attention inputs: dict(lens int32 [B], q bf16 [B, Hq, 128],
    k, v bf16 [B, Tmax, Hkv, 128], pages int32 [B, max_pages] (physical page of
    each logical page, -1 past a sequence's pages), n_pages)."""
    rng = np.random.default_rng(seed)
    lens = rng.integers(lo, hi + 1, size=B).astype(np.int32)
    T = int(lens.max())
    q = to_bf16_tensor(rng.standard_normal((B, Hq, 128)).astype(np.float32))
    k = to_bf16_tensor(rng.standard_normal((B, T, Hkv, 128)).astype(np.float32))
    v = to_bf16_tensor(rng.standard_normal((B, T, Hkv, 128)).astype(np.float32))
    npg = (lens + 15) // 16
    max_pages = int(npg.max())
    n_pages = int(npg.sum()) + extra_pages
    perm = rng.permutation(n_pages).astype(np.int32)
    pages = np.full((B, max_pages), -1, dtype=np.int32)
    o = 0
    for b in range(B):
        pages[b, :npg[b]] = perm[o:o + npg[b]]
        o += npg[b]
    return dict(lens=lens, q=q, k=k, v=v, pages=pages, n_pages=n_pages)
