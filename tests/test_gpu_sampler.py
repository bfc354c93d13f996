"""The denoise loop on the device (flux3_sample, flux3_euler_step) against
the oracle's sample / euler_step / x0_preview.

The Euler update is one fp32 multiply-add per value: its error against the
exact value is at most one rounding of the operands' magnitude,
|got - exact| <= 2^-23 (|x| + |c v|) (fused or not).  The loop is compared on the final latent and
on every step's x0 preview with the transformer-call bar (cosine >= 0.9995,
max-abs <= 3e-2 * max(1, rms(want))).
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


def test_euler_step_with_preview():
    rng = np.random.default_rng(4)
    x = rng.standard_normal(4096 * 128).astype(np.float32)
    v = rng.standard_normal(4096 * 128).astype(np.float32)
    xd, vd = torch.from_numpy(x).to(DEV), torch.from_numpy(v).to(DEV)
    x0 = torch.empty_like(xd)
    s, sn = np.float32(0.8173), np.float32(0.6152)
    F.euler_step(vd, xd, float(s), float(sn), x0_preview=x0)
    torch.cuda.synchronize()
    x64, v64 = x.astype(np.float64), v.astype(np.float64)
    for got, c in ((x0.cpu().numpy(), -float(s)), (xd.cpu().numpy(), float(np.float32(sn - s)))):
        exact = x64 + c * v64
        bound = 2.0 ** -23 * (np.abs(x64) + np.abs(c * v64))
        assert np.all(np.abs(got - exact) <= bound)


def _setup(dims, layout, text_dim, n_pm, n_joint, target, seed=9):
    D = dims.width
    segs = layout.segments()
    modes = sorted({s.mode for s in segs})
    n_text = sum(s.count for s in segs if s.mode == 0)
    n_img = sum(s.count for s in segs if s.mode == 1)
    n_ref = sum(s.count for s in segs if s.mode == 2)
    io = synth.io_weights(seed, D, text_dim=text_dim)
    mw = synth.modulation_weights(seed, D, stages=(0, 1), modes=modes, target=target)
    per_mode = {m: [synth.block_weights(seed, 10 * m + b, dims) for b in range(n_pm)] for m in modes}
    joint = [synth.block_weights(seed, 100 + b, dims) for b in range(n_joint)]
    text, noise, refs = synth.edge_inputs(seed, n_text, n_img, n_ref, text_dim=text_dim)
    return segs, io, mw, per_mode, joint, text, noise, refs


_SMALL_EDIT = synth.RopeLayout(80, 8, 8, ((8, 8),))
SAMPLE_CASES = {
    # width 256, [80 text | 8x8 image | 8x8 reference], 1 + 1 blocks
    "distilled4": (SMALL, 256, _SMALL_EDIT, 4, True),
    "base3": (SMALL, 256, _SMALL_EDIT, 3, False),
    "one_step": (SMALL, 256, _SMALL_EDIT, 1, True),
    # the pages' default: 16 distilled steps ("The denoise loop")
    "distilled16": (SMALL, 256, _SMALL_EDIT, 16, True),
    # model width 3072 with the 20,480-wide text linear, 80 text + 16x16
    # image tokens, 1 + 1 blocks, two distilled steps
    "full_width_distilled2": (synth.DIMS, synth.TEXT_DIM, synth.RopeLayout(80, 16, 16), 2, True),
    # model width, the pages' 16 distilled steps on an edit layout
    # [80 text | 16x16 image | 16x16 reference] (grouped per-mode blocks)
    "full_width_edit_distilled16": (synth.DIMS, synth.TEXT_DIM,
                                    synth.RopeLayout(80, 16, 16, ((16, 16),)), 16, True),
}


@pytest.mark.parametrize("case", sorted(SAMPLE_CASES))
def test_sample_matches_oracle(case):
    dims, text_dim, layout, steps, distilled = SAMPLE_CASES[case]
    segs, io, mw, per_mode, joint, text, noise, refs = _setup(dims, layout, text_dim, 1, 1,
                                                              distilled)
    n = layout.n_tokens
    io_d = {k: bf16_dev(v) for k, v in io.items()}
    mods = []
    for st in (0, 1):
        d = {k: bf16_dev(mw[k]) for k in ("w1", "w2", "w1_tgt", "w2_tgt") if k in mw}
        d["w_mod"] = {m: bf16_dev(v) for m, v in mw["w_mod"][st].items()}
        mods.append(d)
    pm = {m: [upload_weights(w) for w in ws] for m, ws in per_mode.items()}
    jt = [upload_weights(w) for w in joint]
    io_dims = F.IoDims(text_dim, synth.LATENT_DIM)
    lat = torch.from_numpy(noise).to(DEV)
    prev = torch.full((steps,) + noise.shape, float("nan"), dtype=torch.float32, device=DEV)
    ws = torch.empty(F.sample_workspace_bytes(dims, io_dims, n), dtype=torch.uint8, device=DEV)
    F.sample(dims, io_dims, io_d, mods, pm, jt, bf16_dev(text), lat, torch.from_numpy(refs).to(DEV),
             segs, steps, rope_dev(layout), ws, distilled=distilled, previews=prev)
    torch.cuda.synchronize()

    f = synth.bf16_bits_to_f32
    emb = {k: f(mw[k]) for k in ("w1", "w2", "w1_tgt", "w2_tgt") if k in mw}
    w_mod = [{m: f(w) for m, w in mw["w_mod"][st].items()} for st in (0, 1)]
    rope = O.rope_tables(O.token_positions(layout.n_text, layout.grid_h, layout.grid_w,
                                           layout.refs, layout.hw_scale), layout.theta)
    want, want_prev = O.sample(noise, f(text), refs, [(s.start, s.count, s.mode) for s in segs],
                               {k: f(v) for k, v in io.items()}, emb, w_mod, per_mode, joint, rope,
                               steps=steps, distilled=distilled)
    got = lat.cpu().numpy()
    rms = float(np.sqrt(np.mean(want ** 2)))
    assert_close(got, want, f"sample{steps} final", maxabs_tol=3e-2 * max(1.0, rms))
    gp = prev.cpu().numpy()
    for i in range(steps):
        rms = float(np.sqrt(np.mean(want_prev[i] ** 2)))
        assert_close(gp[i], want_prev[i], f"sample{steps} preview {i}", maxabs_tol=3e-2 * max(1.0, rms))
    # the last step lands on sigma = 0: the last preview is the final latent
    np.testing.assert_allclose(gp[-1], got, rtol=0, atol=1e-5)
