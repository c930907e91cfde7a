"""Write the oracle's expected output for the decode-step stack workload
(24 pre-RMSNorm residual SwiGLU blocks, d=2560, ffn=9728, 128x128 block fp8
weights, M=64 rows, then a bf16 head [4096 x 2560]).

Only the CPU oracle and the seeded input generators are used.  Output:
stack_d2560_ffn9728_m64_oracle.npz with
  logits      the head's logits after all 24 blocks (fp64 stored as float32),
  logits_d1   the head's logits after the first block,
  argmax      [25, 64] per-row argmax of the head applied after 0..24 blocks,
  margin      [25, 64] the gap between the two largest logits at each depth.

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


def main():
    wl = synth.WORKLOADS["stack"]
    M = wl.ms[0]
    h = bf16_to_f64(synth.stack_x(wl, M))
    head = bf16_to_f64(synth.stack_head(wl))
    am, mg = [], []

    def record(h):
        lg = ref.head_logits(h, head)
        top2 = np.sort(lg, axis=1)[:, -2:]
        am.append(ref.argmax_rows(lg).astype(np.int32))
        mg.append((top2[:, 1] - top2[:, 0]).astype(np.float32))
        return lg

    record(h)
    t0 = time.time()
    for layer in range(wl.layers):
        wg, wu, wd = synth.stack_layer_weights(wl, layer)
        q = [ref.QWeight(bf16_to_f64(w), "block") for w in (wg, wu, wd)]
        h = ref.stack_layer(h, *q)
        lg = record(h)
        if layer == 0:
            logits_d1 = lg
        print(f"layer {layer} done ({time.time() - t0:.0f} s)", flush=True)
    np.savez_compressed(OUT, logits=lg.astype(np.float32), logits_d1=logits_d1.astype(np.float32),
                        argmax=np.stack(am), margin=np.stack(mg))
    print("wrote", OUT)


if __name__ == "__main__":
    main()
