"""The device calls under HIP graph capture: nothing in a block or stack
call synchronises, allocates or clears memory, so the whole enqueued
sequence can be captured once and replayed.  Each test captures a call,
replays the graph several times with eager work and synchronisation between
the replays (the output overwritten with NaN), and checks every replay
against the eager call bit for bit (the kernels are deterministic).
"""
import numpy as np
import pytest
import torch

import latent_flow_matching_flux_amd as F
import synth

from gpu_util import DEV, rope_dev, upload_weights, workspace
from stack_inputs import stack_inputs

pytestmark = pytest.mark.gpu

SMALL = synth.Dims(width=256, heads=2, head_dim=128, mlp_hidden=384)
# [200 text | 16x16 image | 12x20 reference]: the per-mode stage runs grouped
GROUPED = synth.RopeLayout(200, 16, 16, ((12, 20),))


@pytest.fixture(scope="module", autouse=True)
def _lib():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    F.load()
    F.profile_enable(False)
    yield
    torch.cuda.synchronize()


def _replays_match(call, out, want, reps=3):
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    torch.cuda.synchronize()
    for rep in range(reps):
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = out.cpu()
        assert torch.equal(got, want), f"replay {rep}: max diff " \
            f"{(got - want).abs().nan_to_num(float('inf')).max().item():.3e}"


def test_stack_graph_replays_match_eager():
    dims = SMALL
    segs, pm, jt, x, m1, m2 = stack_inputs(dims, GROUPED, 2, 3, seed=33)
    pm_d = {m: [upload_weights(w) for w in ws] for m, ws in pm.items()}
    jt_d = [upload_weights(w) for w in jt]
    m1d = torch.from_numpy(np.ascontiguousarray(m1)).to(DEV)
    m2d = torch.from_numpy(np.ascontiguousarray(m2)).to(DEV)
    rope = rope_dev(GROUPED)
    ws = workspace(dims, GROUPED.n_tokens)
    x0 = torch.from_numpy(x).to(DEV)
    xe = x0.clone()
    F.stack_forward(dims, pm_d, jt_d, xe, segs, m1d, m2d, rope, ws)
    torch.cuda.synchronize()
    want = xe.cpu()
    assert torch.isfinite(want).all()
    xg = torch.empty_like(x0)

    def call():
        xg.copy_(x0)
        F.stack_forward(dims, pm_d, jt_d, xg, segs, m1d, m2d, rope, ws)

    _replays_match(call, xg, want)


def test_noalloc_block_graph_replays_match_eager():
    """The allocation-free block (its intermediates in the library's fixed
    array) at 1024 tokens, the size it holds."""
    dims = synth.DIMS
    layout = synth.RopeLayout(240, 28, 28)
    segs = layout.segments()
    w = upload_weights(synth.block_weights(35, 0, dims))
    x0 = torch.from_numpy(synth.tokens(35, layout.n_tokens, dims.width)).to(DEV)
    mod = torch.from_numpy(synth.modulation(35, 0, len(segs), dims.width)).to(DEV)
    rope = rope_dev(layout)
    xe = x0.clone()
    F.block_forward_noalloc(dims, w, xe, segs, mod, rope)
    torch.cuda.synchronize()
    want = xe.cpu()
    assert torch.isfinite(want).all()
    xg = torch.empty_like(x0)

    def call():
        xg.copy_(x0)
        F.block_forward_noalloc(dims, w, xg, segs, mod, rope)

    _replays_match(call, xg, want)
