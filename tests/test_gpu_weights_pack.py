"""The packed weight layout (flux3_weights_pack): the copy is bit-exact, and
a block or stack run from packed weights gives bit-identical results to the
Linear-layout run -- the GEMMs load the same values into the same LDS
slots in the same order, only from contiguous 1-KiB blocks.  Parity of the
Linear-layout path with the oracle is covered in test_gpu_parity.py, so
these equalities carry it over to the packed path."""
import numpy as np
import pytest
import torch

import latent_flow_matching_flux_amd as F
import synth

pytestmark = pytest.mark.gpu

from layouts import unpack_rows  # noqa: E402
from gpu_util import DEV, rope_dev, upload_weights, workspace  # noqa: E402

SMALL = synth.Dims(width=256, heads=2, head_dim=128, mlp_hidden=384)


@pytest.fixture(scope="module", autouse=True)
def _lib():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    F.load()
    yield
    torch.cuda.synchronize()


def packed(dims, w_dev):
    buf = torch.empty(F.weights_packed_bytes(dims), dtype=torch.uint8, device=DEV)
    return F.weights_pack(dims, w_dev, buf), buf


def shapes(dims):
    D, Fh = dims.width, dims.mlp_hidden
    return {"wq": (D, D), "wk": (D, D), "wv": (D, D), "wo": (D, D), "w_gate": (Fh, D),
            "w_up": (Fh, D), "w_down": (D, Fh)}


@pytest.mark.parametrize("dims", [SMALL, synth.DIMS], ids=["small", "model"])
def test_pack_copies_every_matrix_exactly(dims):
    w_np = synth.block_weights(0, 3, dims)
    w_dev = upload_weights(w_np)
    pw, buf = packed(dims, w_dev)
    torch.cuda.synchronize()
    assert pw.layout == F.WEIGHTS_PACKED
    base = buf.data_ptr()
    host = buf.cpu().numpy()
    for name, (R, K) in shapes(dims).items():
        off = getattr(pw, name) - base
        assert off % 256 == 0 and 0 <= off and off + R * K * 2 <= buf.numel()
        got = unpack_rows(host[off:off + R * K * 2].view(np.uint16), R, K)
        assert np.array_equal(got, w_np[name]), name
    assert pw.q_norm == w_dev["q_norm"].data_ptr() and pw.k_norm == w_dev["k_norm"].data_ptr()


def _block(dims, w, x0, segs, mod, layout):
    x = x0.clone()
    F.block_forward(dims, w, x, segs, mod, rope_dev(layout), workspace(dims, x.shape[0]))
    torch.cuda.synchronize()
    return x


@pytest.mark.parametrize("name", ["block336", "t2i4336", "permode_text240"])
def test_block_packed_equals_linear(name):
    wl = synth.workload(name)
    dims = synth.DIMS
    layout = wl.layout
    segs = layout.segments()
    n = layout.n_tokens
    w_dev = upload_weights(synth.block_weights(0, 11, dims, norm_stress=True))
    pw, buf = packed(dims, w_dev)
    x0 = torch.from_numpy(synth.tokens(0, n, dims.width)).to(DEV)
    mod = torch.from_numpy(synth.modulation(0, 0, len(segs), dims.width)).to(DEV)
    a = _block(dims, w_dev, x0, segs, mod, layout)
    b = _block(dims, pw, x0, segs, mod, layout)
    assert torch.equal(a, b), f"max diff {(a - b).abs().max().item()}"
    assert not torch.equal(a, x0)


def test_stack_packed_equals_linear():
    dims = SMALL
    layout = synth.RopeLayout(80, 16, 16, ((16, 16),))
    segs = layout.segments()
    n = layout.n_tokens
    lin, pk, bufs = [], [], []
    for b in range(3 * 2 + 2):
        w = upload_weights(synth.block_weights(1, b, dims))
        p, buf = packed(dims, w)
        lin.append(w)
        pk.append(p)
        bufs.append(buf)
    x0 = torch.from_numpy(synth.tokens(1, n, dims.width)).to(DEV)
    m1 = torch.from_numpy(synth.modulation(1, 0, len(segs), dims.width)).to(DEV)
    m2 = torch.from_numpy(synth.modulation(1, 1, len(segs), dims.width)).to(DEV)
    rope = rope_dev(layout)
    outs = []
    for ws_set in (lin, pk):
        x = x0.clone()
        F.stack_forward(dims, ws_set[:6], ws_set[6:], x, segs, m1, m2, rope, workspace(dims, n))
        torch.cuda.synchronize()
        outs.append(x)
    assert torch.equal(outs[0], outs[1])
