"""Device transformer call (flux3_transformer_forward) against the oracle's
transformer_forward: input linears, both stages' modulation from t, the
stack, and the output layer on the image rows.

The oracle runs in float64 on the same bf16 weights and inputs (latent
tokens drawn bf16-representable, so the device's rounding to bf16 is exact).
Bar, as for the stack: cosine >= 0.9995 and max-abs <= 3e-2 * max(1,
rms(want)) on the velocity.  Cases cover the split linear (text projection
of K = 20480 cut into pieces, the 128-row output linear), the direct one
(the K = 128 input linears), several reference segments, and the base and
distilled (target timestep) models, and one call at the model's full width
and depth.
"""
import numpy as np
import pytest
import torch

import latent_flow_matching_flux_amd as F
import synth
from oracle import flux3_oracle as O

pytestmark = pytest.mark.gpu

from gpu_util import DEV, assert_close, bf16_dev, rope_dev, upload_weights  # noqa: E402

SMALL = synth.Dims(width=256, heads=2, head_dim=128, mlp_hidden=384)


@pytest.fixture(scope="module", autouse=True)
def _lib():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    F.load()
    yield
    torch.cuda.synchronize()


def _case(dims, layout, text_dim, n_pm, n_joint, t, t_target, seed=3):
    D = dims.width
    segs = layout.segments()
    n = layout.n_tokens
    modes = sorted({s.mode for s in segs})
    n_text = sum(s.count for s in segs if s.mode == 0)
    n_img = sum(s.count for s in segs if s.mode == 1)
    n_ref = sum(s.count for s in segs if s.mode == 2)
    io = synth.io_weights(seed, D, text_dim=text_dim)
    mw = synth.modulation_weights(seed, D, stages=(0, 1), modes=modes, target=t_target is not None)
    # a full-depth stack cycles through 2 weight sets per mode and 3 joint
    # ones (same composition, bounded host memory and drawing time)
    deep = n_pm + n_joint > 6
    cache = {}

    def bw(block_id):
        if block_id not in cache:
            cache[block_id] = synth.block_weights(seed, block_id, dims)
        return cache[block_id]

    per_mode = {m: [bw(10 * m + (b % 2 if deep else b)) for b in range(n_pm)] for m in modes}
    joint = [bw(100 + (b % 3 if deep else b)) for b in range(n_joint)]
    text, image, refs = synth.edge_inputs(seed, n_text, n_img, n_ref, text_dim=text_dim)

    # device
    io_d = {k: bf16_dev(v) for k, v in io.items()}
    def mod_d(stage):
        out = {k: bf16_dev(mw[k]) for k in ("w1", "w2", "w1_tgt", "w2_tgt") if k in mw}
        out["w_mod"] = {m: bf16_dev(v) for m, v in mw["w_mod"][stage].items()}
        return out
    pm_d = {m: [upload_weights(w) for w in ws] for m, ws in per_mode.items()}
    jt_d = [upload_weights(w) for w in joint]
    text_d = bf16_dev(text) if n_text else None
    img_d = torch.from_numpy(image).to(DEV)
    ref_d = torch.from_numpy(refs).to(DEV) if n_ref else None
    v = torch.full((n_img, synth.LATENT_DIM), float("nan"), dtype=torch.float32, device=DEV)
    io_dims = F.IoDims(text_dim, synth.LATENT_DIM)
    ws = torch.empty(F.transformer_workspace_bytes(dims, io_dims, n), dtype=torch.uint8, device=DEV)
    F.transformer_forward(dims, io_dims, io_d, [mod_d(0), mod_d(1)], pm_d, jt_d, text_d, img_d,
                          ref_d, segs, t, rope_dev(layout), v, ws, t_target=t_target)
    torch.cuda.synchronize()
    got = v.cpu().numpy()

    # oracle
    f = synth.bf16_bits_to_f32
    emb = {k: f(mw[k]) for k in ("w1", "w2", "w1_tgt", "w2_tgt") if k in mw}
    w_mod = [{m: f(w) for m, w in mw["w_mod"][st].items()} for st in (0, 1)]
    rope = O.rope_tables(O.token_positions(layout.n_text, layout.grid_h, layout.grid_w,
                                           layout.refs, layout.hw_scale), layout.theta)
    io_f = {k: f(v_) for k, v_ in io.items()}
    args = (f(text), image, refs, [(s.start, s.count, s.mode) for s in segs], io_f, emb, w_mod,
            per_mode, joint, rope, t)
    want = O.transformer_forward(*args, t_target=t_target)
    floor = None
    if deep:
        # the same call with the stack's blocks rounded to bf16 where the
        # kernels store bf16 (tests/bf16_emulation.py) and nothing else
        # changed: how far bf16 storage alone lands from the oracle
        emu = O.transformer_forward(*args, t_target=t_target, block_fn=_emulated_block())
        floor = float(np.abs(emu - want).max())
    return got, want, floor


def _emulated_block():
    import torch as _t
    from bf16_emulation import _weights, block
    cache = {}

    def fn(xb, wb, sg, md, rp, dtype=np.float64):
        if id(wb) not in cache:
            cache[id(wb)] = _weights(wb)
        with _t.no_grad():
            out = block(_t.from_numpy(np.asarray(xb, np.float32)), cache[id(wb)], sg, md, rp)
        return out.numpy().astype(dtype)
    return fn


def _check(got, want, what, floor=None):
    """The stack bar on the velocity; a full-depth call (floor given) is
    held instead to 1.5 times the bf16-storage floor when that is larger, as
    the full-width 336-token stack is."""
    rms = float(np.sqrt(np.mean(want ** 2)))
    tol = 3e-2 * max(1.0, rms)
    if floor is not None:
        print(f"[floor] {what}: bf16 emulation vs oracle {floor:.4e}")
        tol = max(tol, 1.5 * floor)
    assert_close(got, want, what, maxabs_tol=tol)


CASES = [
    # name, dims, layout, text_dim, n_pm, n_joint, t, t_target
    ("small_two_refs_base", SMALL, synth.RopeLayout(80, 8, 8, ((8, 8), (4, 6))), 256, 1, 2, 0.7,
     None),
    ("small_distilled", SMALL, synth.RopeLayout(80, 8, 12, ((8, 12),)), 512, 2, 1, 0.4, 0.2),
    ("small_no_text", SMALL, synth.RopeLayout(0, 16, 16, ()), 256, 1, 1, 0.9, None),
    ("model_block336", synth.DIMS, synth.RopeLayout(80, 16, 16, ()), synth.TEXT_DIM, 1, 1, 0.55,
     0.3),
    ("model_t2i4336_io_only", synth.DIMS, synth.workload("t2i4336").layout, synth.TEXT_DIM, 0, 0,
     0.8, None),
    # the whole distilled call at the model width and depth (5 per-mode blocks
    # per stream, grouped, then 28 joint) on [80 text | 16x16 image | 16x16
    # reference]
    ("model_edit592_full_depth", synth.DIMS, synth.RopeLayout(80, 16, 16, ((16, 16),)),
     synth.TEXT_DIM, 5, 28, 0.6, 0.45),
    # the 1360 x 768 edit layout (48 x 85 grid and a same-size reference) and
    # ten references, the layouts of "Inside the transformer" / the ten-image
    # reference limit
    ("small_1360x768_edit", SMALL, synth.RopeLayout(240, 48, 85, ((48, 85),)), 256, 1, 1, 0.5,
     0.35),
    ("small_ten_refs", SMALL, synth.RopeLayout(80, 16, 16, tuple((8 + k, 12 - k % 3)
                                                                  for k in range(10))), 256, 1, 1,
     0.65, None),
    # references without text; a ragged grid; t at both ends of the schedule
    ("small_refs_no_text_t1", SMALL, synth.RopeLayout(0, 7, 9, ((5, 3),)), 256, 1, 1, 1.0, 0.99),
    ("small_ragged_t0", SMALL, synth.RopeLayout(13, 5, 11, ()), 256, 1, 1, 0.0, None),
]


@pytest.mark.parametrize("name,dims,layout,text_dim,n_pm,n_joint,t,t_target", CASES,
                         ids=[c[0] for c in CASES])
def test_transformer_matches_oracle(name, dims, layout, text_dim, n_pm, n_joint, t, t_target):
    got, want, floor = _case(dims, layout, text_dim, n_pm, n_joint, t, t_target)
    assert got.shape == want.shape
    _check(got, want, name, floor)


def test_transformer_stage1_velocity_ignores_text_and_refs():
    """Without joint blocks the image velocity is bit-identical whatever the
    text and reference inputs are."""
    dims = SMALL
    layout = synth.RopeLayout(80, 8, 8, ((8, 8),))
    segs = layout.segments()
    n = layout.n_tokens
    io = {k: bf16_dev(v) for k, v in synth.io_weights(5, dims.width, text_dim=256).items()}
    mw = synth.modulation_weights(5, dims.width, stages=(0, 1))
    mods = []
    for st in (0, 1):
        d = {"w1": bf16_dev(mw["w1"]), "w2": bf16_dev(mw["w2"])}
        d["w_mod"] = {m: bf16_dev(v) for m, v in mw["w_mod"][st].items()}
        mods.append(d)
    pm = {m: [upload_weights(synth.block_weights(5, m, dims))] for m in range(3)}
    text, image, refs = synth.edge_inputs(5, 80, 64, 64, text_dim=256)
    io_dims = F.IoDims(256, synth.LATENT_DIM)
    ws = torch.empty(F.transformer_workspace_bytes(dims, io_dims, n), dtype=torch.uint8, device=DEV)
    outs = []
    for k in range(2):
        tx = bf16_dev(text) if k == 0 else bf16_dev(synth.bf16_round_bits(
            synth.bf16_bits_to_f32(text) + 1.0))
        rf = torch.from_numpy(refs * (1.0 + k)).to(DEV)
        v = torch.empty((64, synth.LATENT_DIM), dtype=torch.float32, device=DEV)
        F.transformer_forward(dims, io_dims, io, mods, pm, [], tx, torch.from_numpy(image).to(DEV),
                              rf, segs, 0.6, rope_dev(layout), v, ws)
        torch.cuda.synchronize()
        outs.append(v.cpu().numpy())
    assert np.array_equal(outs[0], outs[1])
    assert np.all(np.isfinite(outs[0]))
