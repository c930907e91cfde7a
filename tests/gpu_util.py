"""Shared helpers of the GPU parity tests (imported by tests only)."""

import sys

import numpy as np
import pytest
import torch

from oracle import ref
from synth import bf16_to_f64

FMT_NAME = {1: "block", 2: "mx"}


def dev():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    return torch.device("cuda:0")


def note(msg):
    """Print and flush a line naming the case about to run on the GPU."""
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def bf16_bits(t):
    return t.detach().cpu().view(torch.int16).numpy().view(np.uint16)


def gpu_out_f64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def assert_close(y_gpu, y_ref, what):
    rf = ref.rel_fro(y_gpu, y_ref)
    ma = ref.max_abs_ratio(y_gpu, y_ref)
    print(f"[parity] {what}: rel_fro={rf:.3e} max_abs_ratio={ma:.3e}", flush=True)
    assert rf <= ref.REL_FRO_TOL, f"{what}: rel_fro {rf:.3e} > {ref.REL_FRO_TOL}"
    assert ma <= ref.MAX_ABS_TOL, f"{what}: max_abs_ratio {ma:.3e} > {ref.MAX_ABS_TOL}"
    return rf, ma


def oracle_weight(w_bf16_cpu, fmt):
    return ref.QWeight(bf16_to_f64(w_bf16_cpu), fmt)
