"""The largest call the library takes: 2^20 tokens, here a 1024 x 1024
image-token grid (twice the 4K layout's side), at the model width.

Rotary tables: every entry bit-exact against the oracle's table (the page's
position table, "prepare_rope_inputs" step of the modular pipeline in the
everytik.com translation of the Diffusers post).

Joint block: every token carries the same input row.  Then every value row
is the same vector v, and softmax attention returns v at every query
whatever its weights are (they sum to one), so each of the 2^20 output rows
equals the oracle's block over that one token alone, whose attention over
its single key is v as well ("Inside the transformer", rohitghumare.com
guide: LayerNorm, attention beside the SwiGLU MLP, gated residual).  Every
row is held to the block tests' bar (max-abs 3e-2, cosine >= 0.9995 on the
output and on its change from the input).  This covers the indexing of all
rows, heads and 16,384 key tiles at the size limit, including buffers past
2^31 elements; what the queries and keys compute leaves no trace in this
case and is checked by the sized parity tests.
"""
import numpy as np
import pytest
import torch

import latent_flow_matching_flux_amd as F
import synth
from oracle import flux3_oracle as O
from synth.configs import MODE_IMAGE

from gpu_util import COS_TOL, DEV, MAXABS_TOL, rope_dev, seg_tuples, upload_weights, workspace

pytestmark = pytest.mark.gpu

N_MAX = 1 << 20
LAYOUT = synth.RopeLayout(0, 1024, 1024, ())
SEED = 47


@pytest.fixture(scope="module", autouse=True)
def _lib():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    F.load()
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _oracle_rope():
    return O.rope_tables(O.token_positions(LAYOUT.n_text, LAYOUT.grid_h, LAYOUT.grid_w,
                                           LAYOUT.refs, LAYOUT.hw_scale), LAYOUT.theta)


@pytest.mark.timeout(300)
def test_rope_tables_max_tokens_bit_exact():
    assert LAYOUT.n_tokens == N_MAX
    got = rope_dev(LAYOUT).cpu().numpy()
    want = _oracle_rope()
    assert got.shape == want.shape == (N_MAX, 64, 2)
    bad = np.argwhere(got.view(np.uint32) != want.view(np.uint32))
    assert bad.size == 0, f"{len(bad)} mismatching entries, first {bad[:5].tolist()}"


@pytest.mark.timeout(300)
def test_block_max_tokens_identical_rows():
    dims = synth.DIMS
    segs = LAYOUT.segments()
    assert seg_tuples(segs) == [(0, N_MAX, MODE_IMAGE)]
    w_np = synth.block_weights(SEED, 0, dims)
    x_row = synth.tokens(SEED, 1, dims.width)
    mod_np = np.ascontiguousarray(synth.modulation(SEED, 1, 1, dims.width), np.float32)
    # the oracle's block over the one token (any rotary row: one key)
    rope_row = _oracle_rope()[:1]
    want = O.block_forward(x_row, w_np, [(0, 1, MODE_IMAGE)], mod_np, rope_row)[0]
    print(f"[max-size] block over {N_MAX} identical tokens, seed {SEED}", flush=True)

    x = torch.from_numpy(x_row).to(DEV).expand(N_MAX, -1).contiguous()
    mod = torch.from_numpy(mod_np).to(DEV)
    rope = rope_dev(LAYOUT)
    ws = workspace(dims, N_MAX)
    F.block_forward(dims, upload_weights(w_np), x, segs, mod, rope, ws)
    torch.cuda.synchronize()
    del ws, rope
    torch.cuda.empty_cache()

    # every row against the one expected row, on the device in row chunks
    want_d = torch.from_numpy(want).to(DEV)                       # fp64 [D]
    x_in = torch.from_numpy(x_row[0].astype(np.float64)).to(DEV)
    dw = want_d - x_in
    worst_abs, worst_row, min_cos, min_dcos = 0.0, -1, 1.0, 1.0
    finite = True
    chunk = 1 << 15
    for r0 in range(0, N_MAX, chunk):
        got = x[r0:r0 + chunk].double()
        finite &= bool(torch.isfinite(got).all())
        err = (got - want_d).abs().amax(dim=1)
        i = int(torch.argmax(err))
        if float(err[i]) > worst_abs:
            worst_abs, worst_row = float(err[i]), r0 + i
        cos = (got @ want_d) / (got.norm(dim=1) * want_d.norm())
        dg = got - x_in
        dcos = (dg @ dw) / (dg.norm(dim=1) * dw.norm())
        min_cos = min(min_cos, float(cos.min()))
        min_dcos = min(min_dcos, float(dcos.min()))
    print(f"[max-size] worst row {worst_row}: max-abs {worst_abs:.3e} (tol {MAXABS_TOL:.0e}), "
          f"min cosine {min_cos:.8f}, min delta cosine {min_dcos:.8f}", flush=True)
    assert finite, "non-finite block output"
    assert worst_abs <= MAXABS_TOL, f"row {worst_row}: max-abs {worst_abs:.3e}"
    assert min_cos >= COS_TOL and min_dcos >= COS_TOL, (min_cos, min_dcos)
