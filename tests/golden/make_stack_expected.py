"""Write the oracle's expected output for the decode-step stack workload
(24 pre-RMSNorm residual SwiGLU blocks, d=2560, ffn=9728, 128x128 block fp8
weights, M=64 rows, then a bf16 head [4096 x 2560]), together with the
spread of equally valid results that the GPU's stack is checked against.

Why a spread.  With random N(0, 0.02) weights each block's output is as large
as the residual stream and fp8 quantization is discontinuous, so the stack
amplifies any difference in rounding: two correct implementations whose fp32
summation orders differ drift apart block by block.  The unperturbed oracle
is one member; the others are the same oracle with seeded one-bf16-ulp
changes planted in block outputs, the kind of difference a different
(correct) summation order makes there:

* family "first": K runs, 1 % of block 0's outputs moved by one bf16 ulp;
* family "every": K runs, 1 % of every block's outputs moved by one ulp (an
  implementation differs from the oracle in every block, not only the first;
  matrix instructions whose internal sums keep fewer bits than fp32 flip the
  bf16 rounding of a few tenths of a percent of a block's outputs).

For each run and each depth (the head applied after 0..24 blocks) the file
records, against the unperturbed oracle: how many rows' argmax agree, the
relative Frobenius error of the logits on a fixed subset of columns (every
8th), the largest |difference| of a logit on that subset, and how many
mismatching rows are NOT near-ties (a near-tie is a row whose oracle margin,
the gap between its two largest logits, is below 4 x that largest
difference).

Only the CPU oracle and the seeded input generators are used.  All runs go
through the oracle together (rows stacked: every step of a block is
row-independent), one layer's weights at a time.  Output:
stack_d2560_ffn9728_m64_oracle.npz with
  logits      the unperturbed logits after all 24 blocks (float32),
  logits_d1   the unperturbed logits after the first block,
  argmax      [25, 64] per-row argmax after 0..24 blocks,
  margin      [25, 64] the gap between the two largest logits,
  cols        the column subset,
  logits_sub  [25, 64, len(cols)] the unperturbed logits on that subset,
  {first,every}_{agree,relerr,maxdiff,nonneartie}  [K, 25] per run and depth.

Run from the repository root:  python tests/golden/make_stack_expected.py
"""
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import synth  # noqa: E402
from oracle import ref  # noqa: E402
from synth import bf16_to_f64  # noqa: E402

OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "stack_d2560_ffn9728_m64_oracle.npz")
K = 32
FAMILIES = {"first": (0.01, "block 0"), "every": (0.01, "every block")}
COL_STRIDE = 8
NEAR_TIE = 4.0


def bump_ulp(y, frac, rng):
    """Move a seeded `frac` of the entries of y (float64 holding bf16 values)
    by one bf16 ulp, up or down at random, through the bf16 bit pattern."""
    y32 = y.astype(np.float32)
    bits = (y32.view(np.uint32) >> 16).astype(np.int64).reshape(-1)
    n = int(round(frac * bits.size))
    idx = rng.choice(bits.size, n, replace=False)
    step = rng.choice(np.array([-1, 1]), n)
    mag = bits[idx] & 0x7FFF
    # one step of the magnitude, never below zero or into inf/NaN
    new = np.clip(mag + step, 0, 0x7F7F)
    bits[idx] = (bits[idx] & 0x8000) | new
    out = (bits.astype(np.uint32) << 16).view(np.float32).reshape(y.shape)
    return out.astype(np.float64)


def compare(lg, base, base_margin, cols):
    """Agreement, relative logit error and max |difference| on the column
    subset, and the number of mismatching rows that are not near-ties."""
    am, am0 = ref.argmax_rows(lg), ref.argmax_rows(base)
    sub, sub0 = lg[:, cols], base[:, cols]
    maxdiff = float(np.max(np.abs(sub - sub0)))
    mism = am != am0
    nonnear = int(np.sum(mism & (base_margin >= NEAR_TIE * maxdiff)))
    return int(np.sum(~mism)), ref.rel_fro(sub, sub0), maxdiff, nonnear


def main():
    wl = synth.WORKLOADS["stack"]
    M = wl.ms[0]
    runs = [("base", 0)] + [(f, k) for f in FAMILIES for k in range(K)]
    R = len(runs)
    x0 = bf16_to_f64(synth.stack_x(wl, M))
    H = np.concatenate([x0] * R, axis=0)  # fp32-exact (bf16 values)
    head = bf16_to_f64(synth.stack_head(wl))
    cols = np.arange(0, wl.vocab, COL_STRIDE)
    rngs = {r: np.random.default_rng(77000 + i) for i, r in enumerate(runs)}
    am, mg, sub = [], [], []
    stats = {f: np.zeros((K, 4, wl.layers + 1)) for f in FAMILIES}

    def record(depth):
        lg = ref.head_logits(H, head)
        base = lg[:M]
        top2 = np.sort(base, axis=1)[:, -2:]
        margin = top2[:, 1] - top2[:, 0]
        am.append(ref.argmax_rows(base).astype(np.int32))
        mg.append(margin.astype(np.float32))
        sub.append(base[:, cols].astype(np.float32))
        for i, (f, k) in enumerate(runs[1:], start=1):
            stats[f][k, :, depth] = compare(lg[i * M:(i + 1) * M], base, margin, cols)
        return base

    record(0)
    t0 = time.time()
    for layer in range(wl.layers):
        wg, wu, wd = synth.stack_layer_weights(wl, layer)
        q = [ref.QWeight(bf16_to_f64(w), "block") for w in (wg, wu, wd)]
        Y = ref.block_output(H, *q)
        for i, (f, k) in enumerate(runs[1:], start=1):
            frac, where = FAMILIES[f]
            if where == "every block" or layer == 0:
                Y[i * M:(i + 1) * M] = bump_ulp(Y[i * M:(i + 1) * M], frac, rngs[(f, k)])
        H = ref.residual_add(H, Y)
        lg = record(layer + 1)
        if layer == 0:
            logits_d1 = lg
        line = " ".join(f"{f}: agree {int(stats[f][:, 0, layer + 1].min())}-{int(stats[f][:, 0, layer + 1].max())} "
                        f"relerr {stats[f][:, 1, layer + 1].max():.2e}" for f in FAMILIES)
        print(f"layer {layer} done ({time.time() - t0:.0f} s)  {line}", flush=True)
    out = dict(logits=lg.astype(np.float32), logits_d1=logits_d1.astype(np.float32),
               argmax=np.stack(am), margin=np.stack(mg), cols=cols, logits_sub=np.stack(sub),
               near_tie_factor=np.float64(NEAR_TIE))
    for f in FAMILIES:
        out[f"{f}_agree"] = stats[f][:, 0].astype(np.int32)
        out[f"{f}_relerr"] = stats[f][:, 1]
        out[f"{f}_maxdiff"] = stats[f][:, 2]
        out[f"{f}_nonneartie"] = stats[f][:, 3].astype(np.int32)
        out[f"{f}_frac"] = np.float64(FAMILIES[f][0])
    np.savez_compressed(OUT, **out)
    print("wrote", OUT)


if __name__ == "__main__":
    main()
