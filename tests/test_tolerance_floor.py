"""Why stack outputs are held to max-abs <= 3e-2 * max(1, rms(x_out)) rather
than a flat 3e-2: any computation that keeps the path's intermediates in
bf16 lands farther than 3e-2 from the fp32 oracle after 33 blocks.

The emulation (tests/bf16_emulation.py) is the oracle's own sequence of
steps with bf16 rounding at exactly the points where the HIP kernels store
bf16 (h, q, k, v, P, o, act) and no other error.  On the 336-token
workload's 5 + 28 stack at the model width -- the same seeded inputs as the
GPU stack test -- it sits above the flat bar while agreeing with the oracle
to a delta cosine far above 0.9995, and inside the rms-scaled bound.  The
residual stream grows (rms ~1.9 after the stack), and bf16 rounding is
relative, so the absolute error grows with it.
"""
import numpy as np
import pytest

import synth
from oracle import flux3_oracle as O

from bf16_emulation import stack as emulated_stack
from stack_inputs import stack_inputs

MAXABS_TOL = 3e-2
COS_TOL = 0.9995


@pytest.mark.slow
def test_stack336_bf16_floor_exceeds_flat_bar():
    dims = synth.DIMS
    layout = synth.workload("block336").layout
    segs, pm, jt, x, m1, m2 = stack_inputs(dims, layout, 5, 28, seed=0)
    st = [(s.start, s.count, s.mode) for s in segs]
    rope = O.rope_tables(O.token_positions(layout.n_text, layout.grid_h, layout.grid_w,
                                           layout.refs, layout.hw_scale), layout.theta)
    want = O.stack_forward(x, pm, jt, st, m1, m2, rope, dtype=np.float32).astype(np.float64)
    emu = emulated_stack(x, pm, jt, st, m1, m2, rope).astype(np.float64)
    floor = float(np.abs(emu - want).max())
    rms = float(np.sqrt(np.mean(want ** 2)))
    dw, de = want - x, emu - x
    cos = float(dw.ravel() @ de.ravel() / (np.linalg.norm(dw) * np.linalg.norm(de)))
    print(f"[floor] bf16 emulation vs fp32 oracle: max-abs {floor:.4e}, rms(x_out) {rms:.3f}, "
          f"delta cosine {cos:.8f}")
    # the flat bar is below what bf16 storage alone produces ...
    assert floor >= MAXABS_TOL
    # ... while the emulation is a faithful computation of the same stack
    assert cos >= COS_TOL
    # and the rms-scaled bound the GPU stack tests use sits above the floor
    assert floor <= MAXABS_TOL * max(1.0, rms)
