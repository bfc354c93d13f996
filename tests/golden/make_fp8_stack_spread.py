"""Writes fp8_stack336_spread.txt: how far the oracle's own rowwise-FP8
stack moves when it is evaluated in float32 instead of float64.

The FP8 block quantises h and [o | act] per token row: a value lying near
the midpoint of two e4m3 codes goes one way or the other depending on the
last bits of the fp32 sums before it.  Over 33 blocks those flipped codes
compound, so two correct evaluations of the same FP8 stack that sum in a
different order land a measurable distance apart.  The GPU's FP8 stack is
held to that spread (tests/test_gpu_fp8.py::test_stack336_full_width).

Inputs: the 336-token workload (80 text + 16 x 16 image), the model dims,
5 per-mode + 28 joint blocks with weights cycling through 2 sets per mode
and 3 joint sets (seed 47), exactly as the GPU test draws them.  Calls only
the oracle.  Run from the repository root:
    python tests/golden/make_fp8_stack_spread.py
"""
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path[:0] = [ROOT, os.path.dirname(HERE)]

import synth  # noqa: E402
from oracle import flux3_oracle as O  # noqa: E402
from stack_inputs import stack_inputs  # noqa: E402

SEED = 47
OUT = os.path.join(HERE, "fp8_stack336_spread.txt")


def main():
    O.THREADS = max(1, min(16, len(os.sched_getaffinity(0))))
    dims = synth.DIMS
    layout = synth.workload("block336").layout
    segs, pm, jt, x, m1, m2 = stack_inputs(dims, layout, 5, 28, seed=SEED)
    st = [(s.start, s.count, s.mode) for s in segs]
    rope = O.rope_tables(O.token_positions(layout.n_text, layout.grid_h, layout.grid_w,
                                           layout.refs, layout.hw_scale), layout.theta)
    q = {}

    def quant(w):
        if id(w) not in q:
            q[id(w)] = O.quantize_block_weights(w)
        return q[id(w)]

    pm_q = {m: [quant(w) for w in ws] for m, ws in pm.items()}
    jt_q = [quant(w) for w in jt]
    out = {}
    for name, dt in (("f32", np.float32), ("f64", np.float64)):
        out[name] = O.stack_forward(x, pm_q, jt_q, st, m1, m2, rope, dtype=dt,
                                    block_fn=O.block_forward_fp8).astype(np.float64)
    a, b = out["f32"], out["f64"]
    x64 = x.astype(np.float64)

    def cos(u, v):
        return float(u.ravel() @ v.ravel() / (np.linalg.norm(u) * np.linalg.norm(v)))

    rows = [("maxabs", float(np.abs(a - b).max())), ("cos_x", cos(a, b)),
            ("cos_delta", cos(a - x64, b - x64)), ("rms_x_out", float(np.sqrt(np.mean(b ** 2))))]
    with open(OUT, "w") as f:
        f.write("# rowwise-FP8 5 + 28 stack, 336 tokens, model dims, seed %d: the oracle in\n"
                "# float32 against the oracle in float64 (written by make_fp8_stack_spread.py)\n"
                % SEED)
        for k, v in rows:
            f.write(f"{k} {v:.9g}\n")
    print(open(OUT).read())


if __name__ == "__main__":
    main()
