"""Seeded inputs of the stack tests, shared by the CPU and the GPU tests.

Block weights cycle through a few distinct sets (2 per mode for the per-mode
stage, 3 for the joint stage by default) so that a 5 + 28 stack at the model
width stays within host memory; the composition is the same as with 43
distinct blocks.
"""
import numpy as np

import synth

_WCACHE = {}


def weights(seed, block_id, dims=synth.DIMS, norm_stress=False):
    key = (seed, block_id, dims, norm_stress)
    if key not in _WCACHE:
        _WCACHE[key] = synth.block_weights(seed, block_id, dims, norm_stress=norm_stress)
    return _WCACHE[key]


def clear_cache():
    _WCACHE.clear()


def stack_inputs(dims, layout, n_pm, n_joint, seed, distinct_pm=2, distinct_joint=3,
                 per_block=False):
    """(segs, per_mode {mode: [w] * n_pm}, joint [w] * n_joint, x, mod_stage1,
    mod_stage2) for the layout's segments."""
    segs = layout.segments()
    n = layout.n_tokens
    pm_np = {m: [weights(seed, 100 + 10 * m + (b % distinct_pm), dims) for b in range(n_pm)]
             for m in range(3)}
    jt_np = [weights(seed, 200 + (b % distinct_joint), dims) for b in range(n_joint)]
    x = synth.tokens(seed, n, dims.width)
    if per_block:
        m1 = np.stack([synth.modulation(seed, 10 + b, len(segs), dims.width) for b in range(n_pm)])
        m2 = np.stack([synth.modulation(seed, 100 + b, len(segs), dims.width) for b in range(n_joint)])
    else:
        m1 = synth.modulation(seed, 1, len(segs), dims.width)
        m2 = synth.modulation(seed, 2, len(segs), dims.width)
    return segs, pm_np, jt_np, x, m1, m2
