"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Bar: RoPE tables bit-exact; block and stack outputs within max-abs 3e-2 and
cosine >= 0.9995 of the oracle, on x_out and on the block delta x_out - x_in
(small gates make x_out ~ x_in, so the delta is where errors show).
"""
import numpy as np
import pytest
import torch

import latent_flow_matching_flux_amd as F
import synth
from oracle import flux3_oracle as O

pytestmark = pytest.mark.gpu

from layouts import unpack_rows  # noqa: E402
from gpu_util import (DEV, assert_close, assert_close_bf16, assert_close_stack,  # noqa: E402
                      bf16_to_np, rope_dev, seg_tuples, upload_weights, vt_unpermute,
                      workspace)

SMALL = synth.Dims(width=256, heads=2, head_dim=128, mlp_hidden=384)


@pytest.fixture(scope="module", autouse=True)
def _lib():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    F.load()
    yield
    torch.cuda.synchronize()


from stack_inputs import stack_inputs as _stack_inputs, weights  # noqa: E402


def run_block(dims, w_np, x_np, segs, mod_np, layout):
    n = x_np.shape[0]
    x = torch.from_numpy(x_np).to(DEV)
    mod = torch.from_numpy(np.ascontiguousarray(mod_np, np.float32)).to(DEV)
    rope = rope_dev(layout)
    ws = workspace(dims, n)
    F.block_forward(dims, upload_weights(w_np), x, segs, mod, rope, ws)
    torch.cuda.synchronize()
    return x.cpu().numpy(), ws, rope


def oracle_rope(layout):
    return O.rope_tables(O.token_positions(layout.n_text, layout.grid_h, layout.grid_w,
                                           layout.refs, layout.hw_scale), layout.theta)


# --------------------------------------------------------------------------
# rotary tables: bit-exact
# --------------------------------------------------------------------------
LAYOUTS = {
    **{k: v.layout for k, v in synth.WORKLOADS.items()},
    "layout_edit_1360x768": synth.RopeLayout(240, 48, 85, ((48, 85),)),
    "ten_refs": synth.RopeLayout(80, 16, 16, tuple((8 + k, 12 - k % 3) for k in range(10))),
    "integer_grid": synth.RopeLayout(80, 16, 16, ((16, 16),), hw_scale=1.0),
}


@pytest.mark.parametrize("name", sorted(LAYOUTS))
def test_rope_tables_bit_exact(name):
    layout = LAYOUTS[name]
    got = rope_dev(layout).cpu().numpy()
    want = oracle_rope(layout)
    assert got.shape == want.shape
    bad = np.argwhere(got.view(np.uint32) != want.view(np.uint32))
    assert bad.size == 0, f"{len(bad)} mismatching entries, first {bad[:5].tolist()}"


# --------------------------------------------------------------------------
# one block, small workload: every intermediate and the output
# --------------------------------------------------------------------------
def _case(name="block336", seed=0, norm_stress=False, dims=synth.DIMS, layout=None):
    layout = layout or synth.workload(name).layout
    n = layout.n_tokens
    segs = layout.segments()
    w = weights(seed, 0, dims, norm_stress)
    x = synth.tokens(seed, n, dims.width)
    mod = synth.modulation(seed, 0, len(segs), dims.width)
    return layout, segs, w, x, mod


@pytest.mark.parametrize("norm_stress", [False, True])
def test_block336_intermediates_and_output(norm_stress):
    dims = synth.DIMS
    layout, segs, w, x, mod = _case(norm_stress=norm_stress)
    n = layout.n_tokens
    got, ws, _ = run_block(dims, w, x, segs, mod, layout)
    want, inter = O.block_forward(x, w, seg_tuples(segs), mod, oracle_rope(layout), keep=True)

    L = F.workspace_layout(dims, n)
    n_pad, D, H, Fh = L.n_pad, dims.width, dims.heads, dims.mlp_hidden
    def view(off, shape):
        nel = int(np.prod(shape))
        return bf16_to_np(ws[off:off + 2 * nel].view(torch.bfloat16).reshape(shape))
    h = unpack_rows(view(L.h, (n_pad * D,)), n_pad, D)[:n]
    q = view(L.q, (H, n_pad, 128))[:, :n].transpose(1, 0, 2)
    k = view(L.k, (H, n_pad, 128))[:, :n].transpose(1, 0, 2)
    vt = vt_unpermute(view(L.vt, (H, 128, n_pad)), n)
    v = vt.transpose(2, 0, 1)
    cat = unpack_rows(view(L.cat, (n_pad * (D + Fh),)), n_pad, D + Fh)[:n]
    assert_close_bf16(h, inter["h"], "K1 h")
    assert_close_bf16(q, inter["q"], "K2 q (RMSNorm+RoPE)")
    assert_close_bf16(k, inter["k"], "K2 k (RMSNorm+RoPE)")
    assert_close_bf16(v, inter["v"], "K2 v")
    assert_close_bf16(cat[:, D:], inter["act"], "K2 silu(gate)*up")
    assert_close_bf16(cat[:, :D], inter["o"], "K3 attention")
    assert_close(got, want, "block x_out")
    assert_close(got - x, want - x, "block delta")
    # padding rows of the workspace hold zeros for q, k, v
    if n_pad > n:
        assert np.all(view(L.k, (H, n_pad, 128))[:, n:] == 0)
        assert np.all(vt_unpermute(view(L.vt, (H, 128, n_pad)), n_pad)[:, :, n:] == 0)


@pytest.mark.parametrize("n_text,grid", [(1, (0, 0)), (7, (0, 0)), (80, (0, 0)), (240, (0, 0)),
                                         (0, (3, 5)), (16, (7, 9)), (80, (17, 19))])
def test_block_ragged_sizes(n_text, grid):
    """Sizes that are not multiples of any tile, single and two segments."""
    dims = synth.DIMS
    layout = synth.RopeLayout(n_text, grid[0], grid[1])
    layout_, segs, w, x, mod = _case(layout=layout, seed=3)
    got, _, _ = run_block(dims, w, x, segs, mod, layout)
    want = O.block_forward(x, w, seg_tuples(segs), mod, oracle_rope(layout))
    assert_close(got, want, f"x_out n={layout.n_tokens}")
    assert_close(got - x, want - x, "delta")


def test_block_small_dims_three_segments():
    dims = SMALL
    layout = synth.RopeLayout(40, 6, 7, ((5, 6),))
    _, segs, w, x, mod = _case(layout=layout, dims=dims, seed=5, norm_stress=True)
    got, _, _ = run_block(dims, w, x, segs, mod, layout)
    want = O.block_forward(x, w, seg_tuples(segs), mod, oracle_rope(layout))
    assert_close(got, want, "x_out small dims")
    assert_close(got - x, want - x, "delta small dims")


def test_gate_zero_is_bit_exact_identity():
    dims = synth.DIMS
    layout, segs, w, x, mod = _case(seed=7)
    mod = mod.copy()
    mod[:, 2] = 0.0
    got, _, _ = run_block(dims, w, x, segs, mod, layout)
    np.testing.assert_array_equal(got, x)


def test_block_is_deterministic():
    dims = synth.DIMS
    layout, segs, w, x, mod = _case(seed=9)
    a, _, _ = run_block(dims, w, x, segs, mod, layout)
    b, _, _ = run_block(dims, w, x, segs, mod, layout)
    np.testing.assert_array_equal(a, b)


def test_error_leaves_x_untouched():
    dims = synth.DIMS
    layout, segs, w, x, mod = _case(seed=11)
    xd = torch.from_numpy(x).to(DEV)
    small_ws = torch.empty(1024, dtype=torch.uint8, device=DEV)
    with pytest.raises(F.Flux3Error) as ei:
        F.block_forward(dims, upload_weights(w), xd, segs,
                        torch.from_numpy(mod).to(DEV), rope_dev(layout), small_ws)
    assert ei.value.status == -5
    torch.cuda.synchronize()
    np.testing.assert_array_equal(xd.cpu().numpy(), x)


# --------------------------------------------------------------------------
# full-size block, edit workload [240 | 4096 | 4096]: every row
# --------------------------------------------------------------------------
def test_block_edit8432_all_rows():
    """The 8432-token joint block the bench times, every row against the
    fp32 oracle."""
    dims = synth.DIMS
    layout, segs, w, x, mod = _case(name="edit8432", seed=0)
    got, _, _ = run_block(dims, w, x, segs, mod, layout)
    want = O.block_forward(x, w, seg_tuples(segs), mod, oracle_rope(layout), dtype=np.float32,
                           attn_chunk=2048)
    assert_close(got, want, "x_out edit8432")
    assert_close(got - x, want - x, "delta edit8432")


# --------------------------------------------------------------------------
# stack
# --------------------------------------------------------------------------
def _run_stack(dims, layout, segs, pm_np, jt_np, x_np, m1, m2, per_block):
    n = x_np.shape[0]
    up = {}
    def dev_w(w):
        k = id(w)
        if k not in up:
            up[k] = upload_weights(w)
        return up[k]
    pm = {m: [dev_w(w) for w in ws] for m, ws in pm_np.items()}
    jt = [dev_w(w) for w in jt_np]
    x = torch.from_numpy(x_np).to(DEV)
    m1d = torch.from_numpy(np.ascontiguousarray(m1, np.float32)).to(DEV)
    m2d = torch.from_numpy(np.ascontiguousarray(m2, np.float32)).to(DEV)
    stride = len(segs) * 3 * dims.width if per_block else 0
    F.stack_forward(dims, pm, jt, x, segs, m1d, m2d, rope_dev(layout), workspace(dims, n),
                    mod_block_stride=stride)
    torch.cuda.synchronize()
    return x.cpu().numpy()


@pytest.mark.parametrize("per_block", [False, True])
def test_stack_small_dims_full_depth(per_block):
    """5 per-mode + 28 joint blocks over [text | image | ref] at reduced width."""
    dims = SMALL
    layout = synth.RopeLayout(48, 8, 10, ((8, 10),))
    segs, pm, jt, x, m1, m2 = _stack_inputs(dims, layout, 5, 28, seed=21, per_block=per_block)
    got = _run_stack(dims, layout, segs, pm, jt, x, m1, m2, per_block)
    want = O.stack_forward(x, pm, jt, seg_tuples(segs), m1, m2, oracle_rope(layout),
                           per_block_mod=per_block)
    assert_close_stack(got, want, x, "stack")


def test_stack_block336_full_dims():
    """5 + 28 blocks at the model width on the 336-token workload (weights
    cycle through 2 sets per mode and 3 joint sets).  Beside the fp32
    oracle, the same stack with bf16 rounding at the kernels' storage points
    and no other error (tests/bf16_emulation.py) gives the floor any bf16
    implementation sits on; the GPU must land within 1.5 times it."""
    from bf16_emulation import stack as emulated_stack
    dims = synth.DIMS
    layout = synth.workload("block336").layout
    segs, pm, jt, x, m1, m2 = _stack_inputs(dims, layout, 5, 28, seed=0)
    got = _run_stack(dims, layout, segs, pm, jt, x, m1, m2, False)
    rope = oracle_rope(layout)
    want = O.stack_forward(x, pm, jt, seg_tuples(segs), m1, m2, rope, dtype=np.float32)
    assert_close_stack(got, want, x, "stack")
    emu = emulated_stack(x, pm, jt, seg_tuples(segs), m1, m2, rope)
    floor = float(np.abs(emu.astype(np.float64) - want).max())
    err = float(np.abs(got.astype(np.float64) - want).max())
    gap = float(np.abs(got.astype(np.float64) - emu).max())
    print(f"[floor] stack336: GPU vs oracle {err:.4e}, bf16 emulation vs oracle {floor:.4e} "
          f"(ratio {err / floor:.3f}), GPU vs emulation {gap:.4e}")
    assert err <= 1.5 * floor


def test_stack_stage1_streams_independent_on_gpu():
    dims = SMALL
    layout = synth.RopeLayout(48, 8, 10, ((8, 10),))
    segs, pm, jt, x, m1, m2 = _stack_inputs(dims, layout, 5, 0, seed=23)
    a = _run_stack(dims, layout, segs, pm, [], x, m1, m2, False)
    x2 = x.copy()
    x2[:48] += 1.0
    b = _run_stack(dims, layout, segs, pm, [], x2, m1, m2, False)
    np.testing.assert_array_equal(a[48:], b[48:])
    assert not np.array_equal(a[:48], b[:48])


# [200 text | 16x16 image | 12x20 reference] = 696 tokens: each stream padded
# to 256 rows fills the 768-row workspace exactly, so the per-mode stage runs
# as one launch sequence per block with a row group per stream; the layout of
# the two tests above (208 tokens, 256 workspace rows) takes one sequence per
# stream instead.
GROUPED = synth.RopeLayout(200, 16, 16, ((12, 20),))


def _stage1_launches(dims, layout, segs, pm, x, m1):
    F.profile_reset()
    F.profile_enable(True)
    try:
        out = _run_stack(dims, layout, segs, pm, [], x, m1, m1, False)
    finally:
        F.profile_enable(False)
    return out, F.profile_read("gemm_proj")["launches"], F.profile_read("attention")["launches"]


def test_stack_stage1_grouped_launch():
    """The per-mode stage as grouped launches: full depth against the
    oracle, streams still independent, and one projection launch per block
    (an attention launch per stream)."""
    dims = SMALL
    segs, pm, jt, x, m1, m2 = _stack_inputs(dims, GROUPED, 5, 2, seed=27)
    got = _run_stack(dims, GROUPED, segs, pm, jt, x, m1, m2, False)
    want = O.stack_forward(x, pm, jt, seg_tuples(segs), m1, m2, oracle_rope(GROUPED))
    assert_close_stack(got, want, x, "grouped stack")
    a, n_proj, n_attn = _stage1_launches(dims, GROUPED, segs, pm, x, m1)
    assert (n_proj, n_attn) == (5, 15)
    x2 = x.copy()
    x2[:200] += 1.0
    b = _run_stack(dims, GROUPED, segs, pm, [], x2, m1, m1, False)
    np.testing.assert_array_equal(a[200:], b[200:])
    assert not np.array_equal(a[:200], b[:200])
    want1 = O.stack_forward(x, pm, [], seg_tuples(segs), m1, m1, oracle_rope(GROUPED))
    assert_close_stack(a, want1, x, "grouped stage 1")


def test_stack_stage1_equal_streams_share_attention():
    """Image and reference streams of equal length attend in one launch
    (heads x streams), each within itself: full depth against the oracle,
    one projection and two attention launches per per-mode block."""
    dims = SMALL
    layout = synth.RopeLayout(200, 16, 16, ((16, 16),))
    segs, pm, jt, x, m1, m2 = _stack_inputs(dims, layout, 5, 2, seed=37)
    got = _run_stack(dims, layout, segs, pm, jt, x, m1, m2, False)
    want = O.stack_forward(x, pm, jt, seg_tuples(segs), m1, m2, oracle_rope(layout))
    assert_close_stack(got, want, x, "equal streams stack")
    a, n_proj, n_attn = _stage1_launches(dims, layout, segs, pm, x, m1)
    assert (n_proj, n_attn) == (5, 10)
    x2 = x.copy()
    x2[200:456] += 1.0                       # the image stream only
    b = _run_stack(dims, layout, segs, pm, [], x2, m1, m1, False)
    np.testing.assert_array_equal(a[:200], b[:200])
    np.testing.assert_array_equal(a[456:], b[456:])
    assert not np.array_equal(a[200:456], b[200:456])


def test_stack_stage1_five_equal_streams_one_attention_launch():
    """[256 text | 16x16 image | three 16x16 references]: five row groups in
    each grouped per-mode launch (the references sharing the reference-mode
    weights), all five streams in one attention launch."""
    dims = SMALL
    layout = synth.RopeLayout(256, 16, 16, ((16, 16), (16, 16), (16, 16)))
    segs, pm, jt, x, m1, m2 = _stack_inputs(dims, layout, 3, 2, seed=41)
    assert [s.count for s in segs] == [256] * 5
    got = _run_stack(dims, layout, segs, pm, jt, x, m1, m2, False)
    want = O.stack_forward(x, pm, jt, seg_tuples(segs), m1, m2, oracle_rope(layout))
    assert_close_stack(got, want, x, "five streams stack")
    _, n_proj, n_attn = _stage1_launches(dims, layout, segs, pm, x, m1)
    assert (n_proj, n_attn) == (3, 3)


def test_stack_grouped_per_block_modulation():
    """Grouped per-mode launches with per-block modulation vectors
    (mod_block_stride): each grouped block reads its own block's vectors
    for every stream."""
    dims = SMALL
    segs, pm, jt, x, m1, m2 = _stack_inputs(dims, GROUPED, 5, 3, seed=39, per_block=True)
    got = _run_stack(dims, GROUPED, segs, pm, jt, x, m1, m2, True)
    want = O.stack_forward(x, pm, jt, seg_tuples(segs), m1, m2, oracle_rope(GROUPED),
                           per_block_mod=True)
    assert_close_stack(got, want, x, "grouped stack, per-block modulation")


def test_stack_stage1_per_stream_fallback_launches():
    """Streams whose padded rows exceed the workspace run one launch
    sequence per stream."""
    dims = SMALL
    layout = synth.RopeLayout(48, 8, 10, ((8, 10),))
    segs, pm, jt, x, m1, m2 = _stack_inputs(dims, layout, 2, 0, seed=29)
    _, n_proj, n_attn = _stage1_launches(dims, layout, segs, pm, x, m1)
    assert (n_proj, n_attn) == (6, 6)


def test_per_mode_block_equals_single_segment_block():
    """A stack with one per-mode block and no joint blocks equals
    block_forward on each stream alone."""
    dims = SMALL
    layout = synth.RopeLayout(48, 8, 10)
    segs, pm, jt, x, m1, m2 = _stack_inputs(dims, layout, 1, 0, seed=25)
    got = _run_stack(dims, layout, segs, pm, [], x, m1, m2, False)
    rope = rope_dev(layout)
    for s_i, s in enumerate(segs):
        xs = torch.from_numpy(x[s.start:s.start + s.count].copy()).to(DEV)
        F.block_forward(dims, upload_weights(pm[s.mode][0]), xs, [(0, s.count, s.mode)],
                        torch.from_numpy(np.ascontiguousarray(m1[s_i:s_i + 1])).to(DEV),
                        rope[s.start:s.start + s.count].contiguous(), workspace(dims, s.count))
        torch.cuda.synchronize()
        np.testing.assert_array_equal(got[s.start:s.start + s.count], xs.cpu().numpy())


# --------------------------------------------------------------------------
# the other workloads: 1024^2 text-to-image block, 4K block, per-mode stage
# --------------------------------------------------------------------------
def test_block_t2i4336_all_rows():
    """One joint block over 240 text + 64x64 image tokens, every row."""
    dims = synth.DIMS
    layout, segs, w, x, mod = _case(name="t2i4336", seed=2)
    got, _, _ = run_block(dims, w, x, segs, mod, layout)
    want = O.block_forward(x, w, seg_tuples(segs), mod, oracle_rope(layout), dtype=np.float32)
    assert_close(got, want, "x_out t2i4336")
    assert_close(got - x, want - x, "delta t2i4336")


def test_block_4k_sampled_rows():
    """One joint block over 240 text + 256x256 image tokens (4096x4096 px):
    the long-sequence attention shape, checked on sampled rows."""
    dims = synth.DIMS
    layout, segs, w, x, mod = _case(name="t2i4k65776", seed=4)
    got, _, _ = run_block(dims, w, x, segs, mod, layout)
    rng = np.random.default_rng(4)
    n = layout.n_tokens
    rows = np.unique(np.concatenate([[0, 239, 240, 241, n - 2, n - 1],
                                     rng.choice(n, 42, replace=False)]))
    want = O.block_forward_rows(x, w, seg_tuples(segs), mod, oracle_rope(layout), rows,
                                dtype=np.float32, attn_chunk=16)
    assert_close(got[rows], want, "x_out rows 4k")
    assert_close(got[rows] - x[rows], want - x[rows], "delta rows 4k")


@pytest.mark.parametrize("name,mode", [("permode_text240", 0), ("permode_image4096", 1)])
def test_per_mode_stage_streams(name, mode):
    """The per-mode stage alone: a stream's 5 blocks with its own weights
    (self-attention within the stream), against the oracle's stack."""
    dims = synth.DIMS
    layout = synth.workload(name).layout
    segs = layout.segments()
    assert len(segs) == 1 and segs[0].mode == mode
    pm = {mode: [weights(7, 300 + b, dims) for b in range(5)]}
    x = synth.tokens(7, layout.n_tokens, dims.width)
    m1 = synth.modulation(7, 3, 1, dims.width)
    got = _run_stack(dims, layout, segs, pm, [], x, m1, m1, False)
    want = O.stack_forward(x, pm, [], seg_tuples(segs), m1, m1, oracle_rope(layout),
                           dtype=np.float32)
    assert_close_stack(got, want, x, f"per-mode {name}")
