"""Rowwise-FP8 blocks (weights of flux3_weights_quantize_fp8r) against the
oracle's FP8 block.

The weight quantisation and the per-token quantisation of [o | act] take
every decision in fp32 on bf16 inputs, as the oracle does, so their codes
and scales are compared bit for bit.  Block and stack outputs are held to
the bf16 bar (max-abs 3e-2, cosine 0.9995) against block_forward_fp8: the
oracle quantises its fp64 h and [o | act], the kernels their fp32 h and
bf16 [o | act], so a code can differ by one step where a value lies next to
a rounding boundary, and the fp8 matrix cores sum with a narrower adder
than fp32 (a few 2^-12 of the largest product of a group).  Over the
full-width 33-block stack those flipped codes compound: that test is held to
the oracle's own float32-against-float64 spread on the same stack."""
import os

import numpy as np
import pytest
import torch

import latent_flow_matching_flux_amd as F
import synth
from oracle import flux3_oracle as O

pytestmark = pytest.mark.gpu

from layouts import unpack8_rows, unpack_rows  # noqa: E402
from gpu_util import (DEV, assert_close, assert_close_stack, bf16_dev, rope_dev,  # noqa: E402
                      seg_tuples, upload_weights, workspace)

SMALL = synth.Dims(width=256, heads=2, head_dim=128, mlp_hidden=384)


@pytest.fixture(scope="module", autouse=True)
def _lib():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    F.load()
    yield
    torch.cuda.synchronize()


def fp8_weights(dims, w_np):
    """Device rowwise-FP8 weights of one block: (BlockWeights, buffer)."""
    w_dev = upload_weights(w_np)
    buf = torch.empty(F.weights_fp8r_bytes(dims), dtype=torch.uint8, device=DEV)
    w8 = F.weights_quantize_fp8r(dims, w_dev, buf)
    w8._keep = (buf, w_dev)
    return w8, buf


_OCACHE = {}


def oracle_fp8(w_np):
    if id(w_np) not in _OCACHE:
        _OCACHE[id(w_np)] = (w_np, O.quantize_block_weights(w_np))
    return _OCACHE[id(w_np)][1]


def _e4m3_decode(codes):
    """Values of e4m3 (FN) codes: sign, 4 exponent bits with bias 7, 3
    mantissa bits; exponent 0 is subnormal (m / 8 * 2^-6); 0x7f / 0xff are
    NaN."""
    c = np.asarray(codes, np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e, m = (c >> 3) & 0xF, c & 0x7
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    return np.where((c & 0x7F) == 0x7F, np.nan, sign * mag)


def _f32_bits(a):
    return np.ascontiguousarray(a, np.float32).view(np.uint32)


def _planted(dims, seed):
    """Block weights with rows that exercise the quantiser's edges: an
    all-zero row, a row of one large value over tiny ones of both signs
    (they round to signed zeros), a row whose maximum is negative, and
    exact ties of the e4m3 grid after scaling."""
    w = {k: np.array(v, copy=True) for k, v in synth.block_weights(seed, 1, dims).items()}
    D = dims.width

    def bits(a):
        return synth.bf16_round_bits(np.asarray(a, np.float32))

    w["wq"][0] = 0
    row = np.full(D, 1e-6, np.float32)
    row[1::2] = -1e-6
    row[7] = 3.0
    w["wq"][1] = bits(row)
    w["wk"][2] = bits(-np.abs(synth.bf16_bits_to_f32(w["wk"][2])) - 0.01)
    # 448 times a tie point between e4m3 values 1.0 and 1.125: with the row
    # maximum 448, the multiplier is exactly 1
    tie = np.linspace(-1, 1, D).astype(np.float32)
    tie[0] = 448.0
    tie[5] = 1.0625
    tie[6] = -1.0625
    tie[9] = 1.1875
    w["w_up"][3] = bits(tie)
    w["w_down"][4] = 0
    w["wo"][4] = 0
    return w


@pytest.mark.parametrize("dims,planted", [(SMALL, True), (synth.DIMS, False)],
                         ids=["small_planted", "model"])
def test_weight_codes_and_scales_bit_exact(dims, planted):
    w_np = _planted(dims, 11) if planted else synth.block_weights(0, 2, dims)
    w8, buf = fp8_weights(dims, w_np)
    torch.cuda.synchronize()
    assert w8.layout == F.WEIGHTS_FP8R
    host = buf.cpu().numpy()
    base = buf.data_ptr()
    D, Fh = dims.width, dims.mlp_hidden

    def codes(name, R, K):
        off = getattr(w8, name) - base
        assert off % 256 == 0 and off + R * K <= host.size
        return unpack8_rows(host[off:off + R * K], R, K)

    def floats(ptr, n):
        off = ptr - base
        return host[off:off + 4 * n].view(np.float32)

    s_proj = floats(w8.s_proj, 3 * D + 2 * Fh)
    row0 = 0
    for name, R in (("wq", D), ("wk", D), ("wv", D), ("w_gate", Fh), ("w_up", Fh)):
        want_c, want_s = O.quantize_rowwise(O.as_float(w_np[name]))
        got_c = codes(name, R, D)
        bad = np.argwhere(got_c != want_c)
        assert bad.size == 0, f"{name}: {len(bad)} codes differ, first {bad[:4].tolist()}"
        np.testing.assert_array_equal(_f32_bits(s_proj[row0:row0 + R]), _f32_bits(want_s))
        row0 += R
    w2 = np.hstack([O.as_float(w_np["wo"]), O.as_float(w_np["w_down"])])
    want_c, want_s = O.quantize_rowwise(w2)
    np.testing.assert_array_equal(codes("wo", D, D), want_c[:, :D])
    np.testing.assert_array_equal(codes("w_down", D, Fh), want_c[:, D:])
    np.testing.assert_array_equal(_f32_bits(floats(w8.s_out, D)), _f32_bits(want_s))
    if planted:
        assert s_proj[0] == 0 and np.all(codes("wq", D, D)[0] == 0)
        assert np.any(codes("wq", D, D)[1] == 0x80)        # negative tiny -> -0
        assert floats(w8.s_out, D)[4] == 0


def _case(layout, seed, dims=synth.DIMS):
    n = layout.n_tokens
    segs = layout.segments()
    w = synth.block_weights(seed, 0, dims)
    x = synth.tokens(seed, n, dims.width)
    mod = synth.modulation(seed, 0, len(segs), dims.width)
    return segs, w, x, mod


def oracle_rope(layout):
    return O.rope_tables(O.token_positions(layout.n_text, layout.grid_h, layout.grid_w,
                                           layout.refs, layout.hw_scale), layout.theta)


def run_fp8_block(dims, w_np, x_np, segs, mod_np, layout):
    n = x_np.shape[0]
    w8, _ = fp8_weights(dims, w_np)
    x = torch.from_numpy(x_np).to(DEV)
    mod = torch.from_numpy(np.ascontiguousarray(mod_np, np.float32)).to(DEV)
    ws = workspace(dims, n)
    F.block_forward(dims, w8, x, segs, mod, rope_dev(layout), ws)
    torch.cuda.synchronize()
    return x.cpu().numpy(), ws


def test_block336_output_and_cat_quantisation():
    """The 336-token block: output against the oracle.  The per-token codes
    and scales of [o | act] that the output GEMM read are checked as a
    property of the device's own buffers, with no oracle involved: each
    row's scale is its largest magnitude / 448 and each code, times that
    scale, is the e4m3 value nearest the bf16 value it encodes.  (The
    quantiser's arithmetic is shared with the weight path, which
    test_weight_codes_and_scales_bit_exact holds bit-exact against the
    oracle on seeded weights.)"""
    dims = synth.DIMS
    layout = synth.workload("block336").layout
    segs, w, x, mod = _case(layout, 0)
    got, ws = run_fp8_block(dims, w, x, segs, mod, layout)
    want = O.block_forward_fp8(x, oracle_fp8(w), seg_tuples(segs), mod, oracle_rope(layout))
    assert_close(got, want, "x_out fp8 block336")
    assert_close(got - x, want - x, "delta fp8 block336")

    n = layout.n_tokens
    L = F.workspace_layout(dims, n)
    n_pad, K = L.n_pad, dims.width + dims.mlp_hidden
    host = ws.cpu().numpy()
    cat = unpack_rows(host[L.cat:L.cat + n_pad * K * 2].view(np.uint16), n_pad, K)[:n]
    vals = (cat.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    got_c = unpack8_rows(host[L.h:L.h + n_pad * K], n_pad, K)[:n]
    s_off = L.h + (n_pad * K + 255) // 256 * 256
    got_s = host[s_off:s_off + 4 * n].view(np.float32).astype(np.float64)
    amax = np.abs(vals).max(axis=1)
    np.testing.assert_allclose(got_s, amax / 448.0, rtol=2 ** -23, atol=0)
    dec = _e4m3_decode(got_c)
    assert np.all(np.isfinite(dec)) and np.abs(dec).max() <= 448.0
    y = vals * (448.0 / np.where(amax > 0, amax, 1.0))[:, None]
    # the nearest grid value: within half a step of the e4m3 grid at y (a
    # hair more for the kernel's fp32 multiplier near a tie)
    step = np.exp2(np.maximum(np.floor(np.log2(np.maximum(np.abs(y), 2.0 ** -9))), -6.0) - 3.0)
    worst = float(np.max(np.abs(dec - y) / step))
    assert worst <= 0.5 + 2 ** -12, f"[o | act] codes: worst |code - value| {worst:.4f} steps"


@pytest.mark.parametrize("n_text,grid", [(1, (0, 0)), (80, (5, 7)), (240, (16, 16))])
def test_block_ragged_sizes(n_text, grid):
    dims = synth.DIMS
    layout = synth.RopeLayout(n_text, grid[0], grid[1])
    segs, w, x, mod = _case(layout, 3)
    got, _ = run_fp8_block(dims, w, x, segs, mod, layout)
    want = O.block_forward_fp8(x, oracle_fp8(w), seg_tuples(segs), mod, oracle_rope(layout))
    assert_close(got, want, f"x_out fp8 n={layout.n_tokens}")
    assert_close(got - x, want - x, "delta fp8")


def test_block_small_dims_three_segments():
    dims = SMALL
    layout = synth.RopeLayout(40, 6, 7, ((5, 6),))
    segs, w, x, mod = _case(layout, 5, dims)
    got, _ = run_fp8_block(dims, w, x, segs, mod, layout)
    want = O.block_forward_fp8(x, oracle_fp8(w), seg_tuples(segs), mod, oracle_rope(layout))
    assert_close(got, want, "x_out fp8 small dims")
    assert_close(got - x, want - x, "delta fp8 small dims")


def test_block_edit8432_all_rows():
    """The 8432-token edit block (the bench's workload), every row."""
    dims = synth.DIMS
    layout = synth.workload("edit8432").layout
    segs, w, x, mod = _case(layout, 0)
    got, _ = run_fp8_block(dims, w, x, segs, mod, layout)
    want = O.block_forward_fp8(x, oracle_fp8(w), seg_tuples(segs), mod, oracle_rope(layout),
                               dtype=np.float32, attn_chunk=2048)
    assert_close(got, want, "x_out fp8 edit8432")
    assert_close(got - x, want - x, "delta fp8 edit8432")


def test_stack_small_dims_full_depth():
    """5 per-mode + 28 joint rowwise-FP8 blocks over [text | image | ref]."""
    dims = SMALL
    layout = synth.RopeLayout(48, 8, 10, ((8, 10),))
    segs = layout.segments()
    n = layout.n_tokens
    pm_np = {m: [synth.block_weights(31 + m, b % 2, dims) for b in range(5)] for m in range(3)}
    jt_np = [synth.block_weights(37, b % 3, dims) for b in range(28)]
    x_np = synth.tokens(31, n, dims.width)
    m1 = synth.modulation(31, 1, len(segs), dims.width)
    m2 = synth.modulation(31, 2, len(segs), dims.width)
    keep = []

    def dev(w):
        w8, buf = fp8_weights(dims, w)
        keep.append((w8, buf))
        return w8

    pm = {m: [dev(w) for w in ws] for m, ws in pm_np.items()}
    jt = [dev(w) for w in jt_np]
    x = torch.from_numpy(x_np).to(DEV)
    F.stack_forward(dims, pm, jt, x, segs,
                    torch.from_numpy(np.ascontiguousarray(m1, np.float32)).to(DEV),
                    torch.from_numpy(np.ascontiguousarray(m2, np.float32)).to(DEV),
                    rope_dev(layout), workspace(dims, n))
    torch.cuda.synchronize()
    got = x.cpu().numpy()
    pm_o = {m: [oracle_fp8(w) for w in ws] for m, ws in pm_np.items()}
    jt_o = [oracle_fp8(w) for w in jt_np]
    want = O.stack_forward(x_np, pm_o, jt_o, seg_tuples(segs), m1, m2, oracle_rope(layout),
                           block_fn=O.block_forward_fp8)
    assert_close_stack(got, want, x_np, "fp8 stack")


def test_stack336_full_width():
    """5 per-mode + 28 joint rowwise-FP8 blocks at the model width on the
    336-token workload (weights cycle through 2 sets per mode and 3 joint
    sets), against the oracle's stack of block_forward_fp8."""
    from stack_inputs import stack_inputs
    dims = synth.DIMS
    layout = synth.workload("block336").layout
    segs, pm_np, jt_np, x_np, m1, m2 = stack_inputs(dims, layout, 5, 28, seed=47)
    n = layout.n_tokens
    dev8 = {}

    def dev(w):
        if id(w) not in dev8:
            dev8[id(w)] = fp8_weights(dims, w)
        return dev8[id(w)][0]

    x = torch.from_numpy(x_np).to(DEV)
    F.stack_forward(dims, {m: [dev(w) for w in ws] for m, ws in pm_np.items()},
                    [dev(w) for w in jt_np], x, segs,
                    torch.from_numpy(np.ascontiguousarray(m1, np.float32)).to(DEV),
                    torch.from_numpy(np.ascontiguousarray(m2, np.float32)).to(DEV),
                    rope_dev(layout), workspace(dims, n))
    torch.cuda.synchronize()
    got = x.cpu().numpy()
    pm_o = {m: [oracle_fp8(w) for w in ws] for m, ws in pm_np.items()}
    jt_o = [oracle_fp8(w) for w in jt_np]
    want = O.stack_forward(x_np, pm_o, jt_o, seg_tuples(segs), m1, m2, oracle_rope(layout),
                           dtype=np.float32, block_fn=O.block_forward_fp8)
    # The bar is the oracle's own spread on this stack (float32 against
    # float64, tests/golden/fp8_stack336_spread.txt): quantisation codes
    # flip with the last bits of the sums before them and the flips compound
    # over 33 blocks, so a correct FP8 stack summed in another order lands
    # about that far away.  The GPU must stay within 1.5 times the spread;
    # the stack without FP8 weights is more than twice as far.
    spread = {}
    with open(os.path.join(os.path.dirname(__file__), "golden", "fp8_stack336_spread.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                k, v = line.split()
                spread[k] = float(v)
    assert_close(got, want, "fp8 stack336 full width x_out",
                 maxabs_tol=1.5 * spread["maxabs"], cos_tol=1 - 1.5 * (1 - spread["cos_x"]))
    assert_close(got - x_np, want - x_np, "fp8 stack336 full width delta",
                 maxabs_tol=1.5 * spread["maxabs"], cos_tol=1 - 1.5 * (1 - spread["cos_delta"]))


def test_block_4k_sampled_rows():
    """The 65,776-token block (240 text + 256 x 256 image tokens): the
    largest configuration, the quantiser over 65,776 rows and K4's
    stream-K tail on fp8 tiles, checked on sampled rows."""
    dims = synth.DIMS
    layout = synth.workload("t2i4k65776").layout
    segs, w, x, mod = _case(layout, 4)
    got, _ = run_fp8_block(dims, w, x, segs, mod, layout)
    rng = np.random.default_rng(4)
    n = layout.n_tokens
    rows = np.unique(np.concatenate([[0, 239, 240, 241, n - 2, n - 1],
                                     rng.choice(n, 26, replace=False)]))
    want = O.block_forward_fp8(x, oracle_fp8(w), seg_tuples(segs), mod, oracle_rope(layout),
                               rows=rows, dtype=np.float32, attn_chunk=16)
    assert_close(got[rows], want, "x_out fp8 rows 4k")
    assert_close(got[rows] - x[rows], want - x[rows], "delta fp8 rows 4k")


def test_transformer_call_with_fp8_blocks():
    """A whole transformer call (input linears, both stages' modulation from
    t, 2 + 2 rowwise-FP8 blocks, the output layer) against the oracle's call
    with its FP8 block; the bar of the bf16 transformer tests."""
    dims = SMALL
    layout = synth.RopeLayout(80, 8, 12, ((8, 12),))
    text_dim, t, t_target, seed = 256, 0.45, 0.25, 8
    D = dims.width
    segs = layout.segments()
    n = layout.n_tokens
    modes = sorted({s_.mode for s_ in segs})
    n_text = sum(s_.count for s_ in segs if s_.mode == 0)
    n_img = sum(s_.count for s_ in segs if s_.mode == 1)
    n_ref = sum(s_.count for s_ in segs if s_.mode == 2)
    io = synth.io_weights(seed, D, text_dim=text_dim)
    mw = synth.modulation_weights(seed, D, stages=(0, 1), modes=modes, target=True)
    per_mode = {m: [synth.block_weights(seed, 10 * m + b, dims) for b in range(2)] for m in modes}
    joint = [synth.block_weights(seed, 100 + b, dims) for b in range(2)]
    text, image, refs = synth.edge_inputs(seed, n_text, n_img, n_ref, text_dim=text_dim)
    keep = []

    def dev(w):
        w8, buf = fp8_weights(dims, w)
        keep.append((w8, buf))
        return w8

    def mod_d(stage):
        out = {k: bf16_dev(mw[k]) for k in ("w1", "w2", "w1_tgt", "w2_tgt")}
        out["w_mod"] = {m: bf16_dev(v) for m, v in mw["w_mod"][stage].items()}
        return out

    io_d = {k: bf16_dev(v) for k, v in io.items()}
    v = torch.full((n_img, synth.LATENT_DIM), float("nan"), dtype=torch.float32, device=DEV)
    io_dims = F.IoDims(text_dim, synth.LATENT_DIM)
    ws = torch.empty(F.transformer_workspace_bytes(dims, io_dims, n), dtype=torch.uint8,
                     device=DEV)
    F.transformer_forward(dims, io_dims, io_d, [mod_d(0), mod_d(1)],
                          {m: [dev(w) for w in ws_] for m, ws_ in per_mode.items()},
                          [dev(w) for w in joint], bf16_dev(text),
                          torch.from_numpy(image).to(DEV), torch.from_numpy(refs).to(DEV), segs,
                          t, rope_dev(layout), v, ws, t_target=t_target)
    torch.cuda.synchronize()
    got = v.cpu().numpy()

    f = synth.bf16_bits_to_f32
    emb = {k: f(mw[k]) for k in ("w1", "w2", "w1_tgt", "w2_tgt")}
    w_mod = [{m: f(w) for m, w in mw["w_mod"][st].items()} for st in (0, 1)]
    want = O.transformer_forward(f(text), image, refs, seg_tuples(segs),
                                 {k: f(v_) for k, v_ in io.items()}, emb, w_mod,
                                 {m: [oracle_fp8(w) for w in ws_] for m, ws_ in per_mode.items()},
                                 [oracle_fp8(w) for w in joint], oracle_rope(layout), t,
                                 t_target=t_target, block_fn=O.block_forward_fp8)
    rms = float(np.sqrt(np.mean(want ** 2)))
    assert_close(got, want, "fp8 transformer velocity", maxabs_tol=3e-2 * max(1.0, rms))


# (layout, per-mode layout of block b for mode m, expected per-mode projection
# launches): streams too long for one grouped launch; streams that fit, with
# one layout per block (grouped launches in each layout); streams that fit
# but whose modes' block-b weights differ in layout (one launch per stream)
MIXED_CASES = {
    "per_stream": (synth.RopeLayout(40, 6, 8, ((6, 8),)), lambda b, m: b, 9),
    "grouped": (synth.RopeLayout(200, 16, 16, ((12, 20),)), lambda b, m: b, 3),
    "modes_differ": (synth.RopeLayout(200, 16, 16, ((12, 20),)), lambda b, m: (b + m) % 3, 9),
}


@pytest.mark.parametrize("case", list(MIXED_CASES))
def test_stack_mixes_weight_layouts(case):
    """One stack whose blocks come in all three layouts (Linear bf16, packed
    bf16, rowwise FP8): each block follows its own weights' arithmetic, in
    grouped per-mode launches or one per stream."""
    dims = SMALL
    layout, kind_of, pm_launches = MIXED_CASES[case]
    segs = layout.segments()
    n = layout.n_tokens
    kinds = ("linear", "packed", "fp8")
    pm_np = {m: [synth.block_weights(51 + m, b, dims) for b in range(3)] for m in range(3)}
    jt_np = [synth.block_weights(57, b, dims) for b in range(3)]
    x_np = synth.tokens(51, n, dims.width)
    m1 = synth.modulation(51, 1, len(segs), dims.width)
    m2 = synth.modulation(51, 2, len(segs), dims.width)
    keep = []

    def dev(w, kind):
        if kind == "fp8":
            w8, buf = fp8_weights(dims, w)
            keep.append((w8, buf))
            return w8
        w_dev = upload_weights(w)
        keep.append(w_dev)
        if kind == "linear":
            return w_dev
        buf = torch.empty(F.weights_packed_bytes(dims), dtype=torch.uint8, device=DEV)
        pw = F.weights_pack(dims, w_dev, buf)
        keep.append((pw, buf))
        return pw

    pm = {m: [dev(w, kinds[kind_of(b, m)]) for b, w in enumerate(ws)] for m, ws in pm_np.items()}
    jt = [dev(w, kinds[(b + 1) % 3]) for b, w in enumerate(jt_np)]
    x = torch.from_numpy(x_np).to(DEV)
    F.profile_reset()
    F.profile_enable(True)
    try:
        F.stack_forward(dims, pm, jt, x, segs,
                        torch.from_numpy(np.ascontiguousarray(m1, np.float32)).to(DEV),
                        torch.from_numpy(np.ascontiguousarray(m2, np.float32)).to(DEV),
                        rope_dev(layout), workspace(dims, n))
        torch.cuda.synchronize()
    finally:
        F.profile_enable(False)
    assert F.profile_read("gemm_proj")["launches"] == pm_launches + 3
    F.profile_reset()
    got = x.cpu().numpy()

    def block(xb, w, sg, md, rp, dtype=np.float64):
        if "w1" in w:
            return O.block_forward_fp8(xb, w, sg, md, rp, dtype=dtype)
        return O.block_forward(xb, w, sg, md, rp, dtype=dtype)

    pm_o = {m: [oracle_fp8(w) if kinds[kind_of(b, m)] == "fp8" else w for b, w in enumerate(ws)]
            for m, ws in pm_np.items()}
    jt_o = [oracle_fp8(w) if kinds[(b + 1) % 3] == "fp8" else w for b, w in enumerate(jt_np)]
    want = O.stack_forward(x_np, pm_o, jt_o, seg_tuples(segs), m1, m2, oracle_rope(layout),
                           block_fn=block)
    assert_close_stack(got, want, x_np, f"mixed-layout stack, {case}")
