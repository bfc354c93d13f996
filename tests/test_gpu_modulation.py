"""Device modulation path against the oracle's modulation_from_t.

Timestep embedding, the two-layer embedder (plus the flow-map target
embedder) and the per-mode modulation linears run as GEMVs over the same
bf16 weights the oracle upcasts; the oracle evaluates them in float64.
The GEMVs accumulate in fp32 over at most 3072 terms, so the bound is
relative to the output scale: max |got - want| <= 1e-4 * max |want| + 1e-7.
"""
import numpy as np
import pytest
import torch

import latent_flow_matching_flux_amd as F
import synth
from oracle import flux3_oracle as O
from gpu_util import DEV, bf16_dev  # noqa: E402

pytestmark = pytest.mark.gpu

SEGS_EDIT = [(0, 240, 0), (240, 4096, 1), (4336, 4096, 2)]
SEGS_T2I = [(0, 240, 0), (240, 4096, 1)]
SEGS_TWO_IMAGE = [(0, 80, 0), (80, 100, 1), (180, 50, 1), (230, 26, 2)]


def _dev_weights(w, stage):
    out = {"w1": bf16_dev(w["w1"]), "w2": bf16_dev(w["w2"])}
    if "w1_tgt" in w:
        out["w1_tgt"] = bf16_dev(w["w1_tgt"])
        out["w2_tgt"] = bf16_dev(w["w2_tgt"])
    out["w_mod"] = {m: bf16_dev(v) for m, v in w["w_mod"][stage].items()}
    return out


def _oracle(w, stage, t_by_mode, modes, t_target):
    f = synth.bf16_bits_to_f32
    kw = {}
    if t_target is not None:
        kw = dict(t_target=t_target, w1_tgt=f(w["w1_tgt"]), w2_tgt=f(w["w2_tgt"]))
    return O.modulation_from_t({m: t_by_mode[m] for m in modes}, f(w["w1"]), f(w["w2"]),
                               {m: f(w["w_mod"][stage][m]) for m in modes}, **kw)


CASES = [
    # name, width, segments, stage, t_by_mode (text, image, ref), t_target
    ("edit8432", 3072, SEGS_EDIT, 0, (0.0, 0.37, 0.0), None),
    ("edit8432_distilled", 3072, SEGS_EDIT, 1, (0.0, 0.37, 0.0), 0.1),
    ("t2i4336_stage2", 3072, SEGS_T2I, 1, (0.0, 0.81, 0.0), None),
    ("three_timesteps_and_target", 3072, SEGS_EDIT, 0, (0.2, 0.6, 0.9), 0.05),
    ("two_image_segments", 256, SEGS_TWO_IMAGE, 0, (0.0, 0.5, 0.0), None),
    ("width_512_t1", 512, SEGS_T2I, 1, (0.0, 1.0, 0.0), 0.0),
]


@pytest.mark.parametrize("name,width,segs,stage,t_by_mode,t_target", CASES,
                         ids=[c[0] for c in CASES])
def test_modulation_matches_oracle(name, width, segs, stage, t_by_mode, t_target):
    dims = synth.Dims(width, width // 128, 128, 3 * width)
    modes = sorted({m for _, _, m in segs})
    w = synth.modulation_weights(7, width, stages=(stage,), modes=modes,
                                 target=t_target is not None)
    wd = _dev_weights(w, stage)
    mod = torch.full((len(segs), 3, width), float("nan"), dtype=torch.float32, device=DEV)
    ws = torch.empty(F.modulation_workspace_bytes(dims), dtype=torch.uint8, device=DEV)
    print(f"[modulation] case {name}: width {width}, segments {segs}, t {t_by_mode}, target {t_target}",
          flush=True)
    F.modulation_forward(dims, wd, t_by_mode, segs, mod, ws, t_target=t_target)
    torch.cuda.synchronize()
    got = mod.cpu().numpy().astype(np.float64)
    want = _oracle(w, stage, t_by_mode, modes, t_target)
    for i, (_, _, m) in enumerate(segs):
        err = float(np.max(np.abs(got[i] - want[m])))
        scale = float(np.max(np.abs(want[m])))
        print(f"[parity] modulation {name} segment {i} (mode {m}): max-abs {err:.3e}, "
              f"scale {scale:.3e}", flush=True)
        assert np.all(np.isfinite(got[i]))
        assert scale > 1e-6
        assert err <= 1e-4 * scale + 1e-7, f"segment {i}: {err:.3e} vs scale {scale:.3e}"


def test_modulation_text_and_reference_do_not_move_with_image_t():
    """The t = 0 path on the device: text and reference vectors are
    bit-identical when only the image timestep changes."""
    dims = synth.DIMS
    w = synth.modulation_weights(11, dims.width)
    wd = _dev_weights(w, 0)
    ws = torch.empty(F.modulation_workspace_bytes(dims), dtype=torch.uint8, device=DEV)
    outs = []
    for t_img in (0.2, 0.9):
        mod = torch.empty((3, 3, dims.width), dtype=torch.float32, device=DEV)
        F.modulation_forward(dims, wd, (0.0, t_img, 0.0), SEGS_EDIT, mod, ws)
        outs.append(mod.cpu().numpy())
    assert np.array_equal(outs[0][0], outs[1][0])
    assert np.array_equal(outs[0][2], outs[1][2])
    assert not np.allclose(outs[0][1], outs[1][1])
