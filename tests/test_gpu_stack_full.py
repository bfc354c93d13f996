"""The full 5 + 28 stack at the configurations the pages time, every row,
against the fp32 oracle: the 1024^2 text-to-image call [240 text | 64x64
image] = 4336 tokens, and the single-reference edit [240 | 4096 | 4096] =
8432 tokens that the bench times ("Speed, architecture, and how the tokens
move", 15jq.com post: 5 per-mode blocks per stream, then 28 joint blocks
over the concatenation).

Weights cycle through 2 sets per mode and 3 joint sets (seeded, recorded
below) so host and device memory stay bounded; every block still runs the
full model width.  Bound: the stack bar of the other stack tests (cosine >=
0.9995 on x_out and on x_out - x_in, max-abs <= 3e-2 * max(1, rms(x_out)),
the rms-scaled bound that tests/test_tolerance_floor.py shows is above the
bf16 storage floor).  Each takes a few minutes of host time for the oracle.
"""
import time

import numpy as np
import pytest
import torch

import latent_flow_matching_flux_amd as F
import synth
from oracle import flux3_oracle as O

from gpu_util import (DEV, assert_close, assert_close_stack, rope_dev, seg_tuples, upload_weights,
                      workspace)
from stack_inputs import clear_cache, stack_inputs

pytestmark = pytest.mark.gpu

SEEDS = {"t2i4336": 41, "edit8432": 43}


@pytest.fixture(scope="module", autouse=True)
def _lib():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    F.load()
    yield
    torch.cuda.synchronize()
    clear_cache()


def _f32(w):
    """The oracle's own widening of a block's bf16 weights, done once per
    distinct set instead of once per block."""
    return {k: O.as_float(v, np.float32) for k, v in w.items()}


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["t2i4336", "edit8432"])
def test_full_stack_all_rows(name):
    dims = synth.DIMS
    layout = synth.workload(name).layout
    seed = SEEDS[name]
    segs, pm, jt, x, m1, m2 = stack_inputs(dims, layout, 5, 28, seed=seed)
    print(f"[stack] {name}: {layout.n_tokens} tokens, seed {seed}, segments "
          f"{seg_tuples(segs)}", flush=True)

    dev = {}

    def dev_w(w):
        if id(w) not in dev:
            dev[id(w)] = upload_weights(w)
        return dev[id(w)]

    n = layout.n_tokens
    xd = torch.from_numpy(x).to(DEV)
    F.stack_forward(dims, {m: [dev_w(w) for w in ws] for m, ws in pm.items()},
                    [dev_w(w) for w in jt], xd, segs,
                    torch.from_numpy(np.ascontiguousarray(m1)).to(DEV),
                    torch.from_numpy(np.ascontiguousarray(m2)).to(DEV), rope_dev(layout),
                    workspace(dims, n))
    torch.cuda.synchronize()
    got = xd.cpu().numpy()
    del dev, xd
    torch.cuda.empty_cache()

    t0 = time.time()
    wide = {}

    def wf(w):
        if id(w) not in wide:
            wide[id(w)] = _f32(w)
        return wide[id(w)]

    rope = O.rope_tables(O.token_positions(layout.n_text, layout.grid_h, layout.grid_w,
                                           layout.refs, layout.hw_scale), layout.theta)
    want = O.stack_forward(x, {m: [wf(w) for w in ws] for m, ws in pm.items()},
                           [wf(w) for w in jt], seg_tuples(segs), m1, m2, rope,
                           dtype=np.float32)
    print(f"[stack] {name}: oracle {time.time() - t0:.1f} s on {O.THREADS} threads", flush=True)
    assert_close_stack(got, want, x, f"stack {name}")


@pytest.mark.timeout(900)
def test_stack_t2i4k65776_composition():
    """The 5 + 28 stack at 65,776 tokens [240 text | 256x256 image] (4096^2
    px), where an oracle stack does not finish in test time.  Checked
    instead: (1) the stack call equals its blocks enqueued one at a time (5
    stack calls of one per-mode block, then 28 block calls) bit for bit, so
    it runs every block in order with its weights and modulation; (2) the
    first per-mode block -- both streams in one grouped launch -- given the
    stack's seeded input, matches the oracle's per-stream block on every
    text row and on sampled image rows; (3) the last joint block's weights
    and modulation, run as one block call on the same seeded input, match
    the oracle's joint block on sampled rows of the whole sequence (every
    oracle input is the seeded one, none comes from the device)."""
    dims = synth.DIMS
    layout = synth.workload("t2i4k65776").layout
    n = layout.n_tokens
    seed = 45
    segs, pm, jt, x, m1, m2 = stack_inputs(dims, layout, 5, 28, seed=seed)
    print(f"[stack] t2i4k65776: {n} tokens, seed {seed}, segments {seg_tuples(segs)}", flush=True)
    dev = {}

    def dev_w(w):
        if id(w) not in dev:
            dev[id(w)] = upload_weights(w)
        return dev[id(w)]

    pm_d = {m: [dev_w(w) for w in ws] for m, ws in pm.items()}
    jt_d = [dev_w(w) for w in jt]
    m1d = torch.from_numpy(np.ascontiguousarray(m1)).to(DEV)
    m2d = torch.from_numpy(np.ascontiguousarray(m2)).to(DEV)
    rope = rope_dev(layout)
    ws = workspace(dims, n)
    x0 = torch.from_numpy(x).to(DEV)

    xs = x0.clone()
    F.stack_forward(dims, pm_d, jt_d, xs, segs, m1d, m2d, rope, ws)
    torch.cuda.synchronize()
    got_stack = xs.cpu().numpy()
    del xs

    xl = x0.clone()
    F.block_forward(dims, jt_d[27], xl, segs, m2d, rope, ws)
    torch.cuda.synchronize()
    got_last = xl.cpu().numpy()
    del xl

    xc = x0.clone()
    x_after_pm0 = None
    for b in range(5):
        F.stack_forward(dims, {m: [ws_[b]] for m, ws_ in pm_d.items()}, [], xc, segs, m1d, m2d,
                        rope, ws)
        if b == 0:
            torch.cuda.synchronize()
            x_after_pm0 = xc.cpu().numpy()
    for b in range(28):
        F.block_forward(dims, jt_d[b], xc, segs, m2d, rope, ws)
    torch.cuda.synchronize()
    got_chain = xc.cpu().numpy()
    del xc, x0, ws, dev, pm_d, jt_d
    torch.cuda.empty_cache()
    assert np.all(np.isfinite(got_stack))
    np.testing.assert_array_equal(got_stack, got_chain)

    t0 = time.time()
    rope_o = O.rope_tables(O.token_positions(layout.n_text, layout.grid_h, layout.grid_w,
                                             layout.refs, layout.hw_scale), layout.theta)
    rng = np.random.default_rng(seed)
    n_text = segs[0].count
    # first per-mode block: each stream alone, from the stack's input
    text_rows = np.arange(n_text)
    want = O.block_forward_rows(x[:n_text], _f32(pm[0][0]), [(0, n_text, 0)], m1[0:1],
                                rope_o[:n_text], text_rows, dtype=np.float32, attn_chunk=16)
    assert_close(x_after_pm0[:n_text], want, "t2i4k65776 per-mode block 0, text rows")
    n_img = n - n_text
    img_rows = np.unique(np.concatenate([[0, 1, 255, 256, n_img - 1],
                                         rng.choice(n_img, 27, replace=False)]))
    want = O.block_forward_rows(x[n_text:], _f32(pm[1][0]), [(0, n_img, 1)], m1[1:2],
                                rope_o[n_text:], img_rows, dtype=np.float32, attn_chunk=16)
    assert_close(x_after_pm0[n_text + img_rows], want, "t2i4k65776 per-mode block 0, image rows")
    # the last joint block's weights over the whole sequence, from the seeded input
    rows = np.unique(np.concatenate([[0, n_text - 1, n_text, n - 1],
                                     rng.choice(n, 28, replace=False)]))
    want = O.block_forward_rows(x, _f32(jt[27]), seg_tuples(segs), m2, rope_o, rows,
                                dtype=np.float32, attn_chunk=16)
    assert_close(got_last[rows], want, "t2i4k65776 joint block 27, sampled rows")
    assert_close(got_last[rows] - x[rows], want - x[rows], "t2i4k65776 joint block 27 delta")
    print(f"[stack] t2i4k65776: oracle rows {time.time() - t0:.1f} s on {O.THREADS} threads",
          flush=True)
