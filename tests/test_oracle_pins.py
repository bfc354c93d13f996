"""Pins for the CPU oracle: checks against what the release pages and the
mathematics fix, independent of the oracle's own code path.

Each test names the fact it pins.  The library routines used as independent
references (torch CPU layer_norm, rms_norm, scaled_dot_product_attention,
silu; complex exponentials) are separate implementations of the textbook
definitions; brute-force loops run on tiny shapes only.
"""
import cmath
import math
import os

import numpy as np
import pytest
import torch

from oracle import flux3_oracle as O
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
RNG = np.random.default_rng(1234)


def _rand(*shape):
    return RNG.standard_normal(shape)


# --------------------------------------------------------------------------
# positions and token counts
# --------------------------------------------------------------------------
def test_positions_match_page_table():
    """Position ids follow the RoPE table (text along l, image and reference on
    the shared (h, w) grid, reference at l = -(k+1))."""
    want = np.loadtxt(os.path.join(GOLDEN, "positions_small.txt"))
    got = O.token_positions(3, 2, 3, refs=((2, 2),))
    np.testing.assert_array_equal(got, want)


def test_positions_several_refs_offset_negatively():
    pos = O.token_positions(0, 1, 1, refs=((1, 1), (1, 1), (1, 1)))
    assert list(pos[:, 3]) == [0.0, -1.0, -2.0, -3.0]


def test_token_counts_match_pages():
    """1024 px -> 64x64 = 4096 tokens; 4096 px -> 65536; one 1024 px reference
    adds 4096 tokens (16x16 px per token)."""
    assert synth.workload("t2i4336").layout.n_image == (1024 // 16) ** 2 == 4096
    assert synth.workload("t2i4k65776").layout.n_image == (4096 // 16) ** 2 == 65536
    assert synth.workload("edit8432").n_tokens - synth.workload("t2i4336").n_tokens == 4096
    for name in ("block336", "t2i4336", "edit8432", "t2i4k65776"):
        assert synth.workload(name).layout.n_text % 80 == 0   # padded to 80s


def test_parameter_count_fits_published_totals():
    """The block shapes (D=3072, 24x128 heads, SwiGLU 9216, q/k norm [128], no
    biases, 43 distinct blocks) reproduce the published base and distilled
    parameter counts exactly together with the input/output/modulation
    linears; the distilled extra is one 256->D->D embedder."""
    d = synth.DIMS
    D, F, hd = d.width, d.mlp_hidden, d.head_dim
    per_block = 4 * D * D + 3 * D * F + 2 * hd
    base = 43 * per_block + 20480 * D + (256 * D + D * D) + 20 * D * D + 3 * 128 * D
    assert base == 5_538_458_368
    assert base + 256 * D + D * D == 5_548_681_984
    assert 256 * 3072 + 3072 * 3072 == 10_223_616


# --------------------------------------------------------------------------
# rotary tables and rotation
# --------------------------------------------------------------------------
def test_rope_table_known_values():
    """Closed forms: the l-axis pair j of text token i has angle
    i * 10000**(-j/16); the t axis never rotates (t = 0 for every token)."""
    pos = O.token_positions(5, 0, 0)
    tab = O.rope_tables(pos)
    assert tab.dtype == np.float32 and tab.shape == (5, 64, 2)
    assert np.all(tab[:, 0:16, 0] == 1.0) and np.all(tab[:, 0:16, 1] == 0.0)
    assert tab[3, 48, 0] == np.float32(math.cos(3.0))
    assert tab[3, 48, 1] == np.float32(math.sin(3.0))
    assert tab[2, 56, 1] == np.float32(math.sin(2.0 * 0.01))   # j=8: 1e4**-0.5
    # text tokens sit at h = w = 0
    assert np.all(tab[:, 16:48, 0] == 1.0) and np.all(tab[:, 16:48, 1] == 0.0)


def test_rope_table_vs_complex_exponential():
    pos = O.token_positions(7, 3, 4, refs=((2, 3),))
    tab = O.rope_tables(pos).astype(np.float64)
    for n in range(pos.shape[0]):
        for p in range(64):
            a, j = divmod(p, 16)
            z = cmath.exp(1j * pos[n, a] * 10000.0 ** (-j / 16.0))
            assert abs(tab[n, p, 0] - z.real) <= 6e-8
            assert abs(tab[n, p, 1] - z.imag) <= 6e-8


def _rot(x, pos, theta=O.THETA):
    """Rotate [N][H][128] by exact fp64 angles (tables not rounded)."""
    pos = np.asarray(pos, float)
    ang = np.zeros((pos.shape[0], 64))
    for p in range(64):
        a, j = divmod(p, 16)
        ang[:, p] = pos[:, a] * theta ** (-2.0 * j / 32)
    tab = np.stack([np.cos(ang), np.sin(ang)], axis=-1)
    return O.apply_rope(x, tab)


def test_rope_rotation_is_complex_multiplication():
    """Pair (x0, x1) rotated by angle phi equals (x0 + i x1) * e^{i phi}."""
    x = _rand(3, 2, 128)
    pos = O.token_positions(1, 1, 2)
    y = _rot(x, pos)
    for n in range(3):
        for hh in range(2):
            for p in range(64):
                a, j = divmod(p, 16)
                z = complex(x[n, hh, 2 * p], x[n, hh, 2 * p + 1]) * cmath.exp(
                    1j * pos[n, a] * 10000.0 ** (-j / 16.0))
                assert abs(y[n, hh, 2 * p] - z.real) < 1e-12
                assert abs(y[n, hh, 2 * p + 1] - z.imag) < 1e-12


def test_rope_preserves_pair_norms():
    x = _rand(40, 3, 128)
    pos = O.token_positions(8, 4, 4, refs=((4, 4),))
    y = O.apply_rope(x, O.rope_tables(pos))
    nx = x[..., 0::2] ** 2 + x[..., 1::2] ** 2
    ny = y[..., 0::2] ** 2 + y[..., 1::2] ** 2
    np.testing.assert_allclose(ny, nx, rtol=2e-7)           # fp32 table
    y64 = _rot(x, pos)
    ny64 = y64[..., 0::2] ** 2 + y64[..., 1::2] ** 2
    np.testing.assert_allclose(ny64, nx, rtol=1e-14)        # exact angles


def test_rope_scores_depend_only_on_position_difference():
    """<R(p)q, R(p')k> is unchanged when every position moves by the same c."""
    pos = O.token_positions(8, 2, 4, refs=((2, 2),))
    q = _rand(pos.shape[0], 1, 128)
    k = _rand(pos.shape[0], 1, 128)
    c = np.array([0.0, 3.5, -2.0, 7.0])
    s0 = _rot(q, pos)[:, 0] @ _rot(k, pos)[:, 0].T
    s1 = _rot(q, pos + c)[:, 0] @ _rot(k, pos + c)[:, 0].T
    np.testing.assert_allclose(s1, s0, rtol=0, atol=1e-10)


def test_rope_axis_ownership():
    """Text tokens rotate only dims 96..127 (l axis); noisy-image tokens only
    dims 32..95 (h, w); an image and a reference token at the same grid spot
    differ only in the l axis, by exactly 1."""
    x = _rand(1, 1, 128)
    text = O.token_positions(4, 0, 0)[3:4]
    y = _rot(x, text)
    np.testing.assert_array_equal(y[..., :96], x[..., :96])
    assert not np.allclose(y[..., 96:], x[..., 96:])
    pos = O.token_positions(0, 3, 3, refs=((3, 3),))
    img, ref = pos[4:5], pos[9 + 4:9 + 5]
    yi = _rot(x, img)
    np.testing.assert_array_equal(yi[..., :32], x[..., :32])
    np.testing.assert_array_equal(yi[..., 96:], x[..., 96:])
    assert np.array_equal(img[:, :3], ref[:, :3]) and ref[0, 3] - img[0, 3] == -1


def test_rope_zero_position_is_identity():
    x = _rand(2, 2, 128)
    y = O.apply_rope(x, O.rope_tables(np.zeros((2, 4))))
    np.testing.assert_array_equal(y, x)


# --------------------------------------------------------------------------
# norms, modulation, activation
# --------------------------------------------------------------------------
def test_layer_norm_moments_and_torch():
    x = _rand(6, 3072) * 3 + 1.5
    y = O.layer_norm(x)
    np.testing.assert_allclose(y.mean(-1), 0, atol=1e-12)
    np.testing.assert_allclose(y.var(-1), 1, rtol=1e-5)     # eps = 1e-6
    t = torch.nn.functional.layer_norm(torch.from_numpy(x), (3072,), eps=1e-6).numpy()
    np.testing.assert_allclose(y, t, rtol=1e-10, atol=1e-12)


def test_modulate_special_cases():
    h = _rand(4, 16)
    z = np.zeros(16)
    np.testing.assert_array_equal(O.modulate(h, z, z), h)
    s = _rand(16)
    np.testing.assert_array_equal(O.modulate(h, s, -np.ones(16)), np.broadcast_to(s, h.shape))
    np.testing.assert_allclose(O.modulate(h, z, np.ones(16)), 2 * h)


def test_rms_norm_heads_unit_rms_and_torch():
    x = _rand(5, 24, 128) * 4
    w = 1 + 0.1 * _rand(128)
    y = O.rms_norm_heads(x, np.ones(128))
    np.testing.assert_allclose(np.sqrt((y ** 2).mean(-1)), 1, rtol=1e-6)
    t = torch.nn.functional.rms_norm(torch.from_numpy(x), (128,), torch.from_numpy(w), eps=1e-6)
    np.testing.assert_allclose(O.rms_norm_heads(x, w), t.numpy(), rtol=1e-12, atol=1e-12)


def test_silu_and_swiglu_vs_torch():
    z = _rand(100) * 5
    np.testing.assert_allclose(O.silu(z), torch.nn.functional.silu(torch.from_numpy(z)).numpy(), rtol=1e-12)
    h, wg, wu, wd = _rand(3, 8), _rand(5, 8), _rand(5, 8), _rand(8, 5)
    th = torch.from_numpy
    ref = (torch.nn.functional.silu(th(h) @ th(wg).T) * (th(h) @ th(wu).T)) @ th(wd).T
    np.testing.assert_allclose(O.swiglu_mlp(h, wg, wu, wd), ref.numpy(), rtol=1e-12)
    # the silu is on the gate branch: swapping gate and up changes the result
    assert not np.allclose(O.swiglu_mlp(h, wu, wg, wd), ref.numpy())


# --------------------------------------------------------------------------
# attention
# --------------------------------------------------------------------------
def _attention_loops(q, k, v):
    n, H, d = q.shape
    out = np.zeros_like(q)
    for h in range(H):
        for i in range(n):
            logits = [sum(q[i, h, c] * k[j, h, c] for c in range(d)) / math.sqrt(d)
                      for j in range(k.shape[0])]
            mx = max(logits)
            w = [math.exp(s - mx) for s in logits]
            tot = sum(w)
            for c in range(d):
                out[i, h, c] = sum(w[j] * v[j, h, c] for j in range(k.shape[0])) / tot
    return out


def test_attention_brute_force_tiny():
    q, k, v = _rand(5, 2, 128), _rand(7, 2, 128), _rand(7, 2, 128)
    np.testing.assert_allclose(O.attention(q, k, v), _attention_loops(q, k, v), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(O.attention(q, k, v, chunk=2), _attention_loops(q, k, v), rtol=1e-12, atol=1e-13)


def test_attention_vs_torch_sdpa():
    q, k, v = _rand(33, 3, 128), _rand(33, 3, 128), _rand(33, 3, 128)
    th = lambda a: torch.from_numpy(a).permute(1, 0, 2).contiguous()  # [H][N][d]
    ref = torch.nn.functional.scaled_dot_product_attention(th(q), th(k), th(v)).permute(1, 0, 2).numpy()
    np.testing.assert_allclose(O.attention(q, k, v), ref, rtol=1e-10, atol=1e-12)


def test_attention_special_cases():
    n = 9
    v = _rand(n, 1, 128)
    # q = 0: uniform average of v
    out = O.attention(np.zeros((3, 1, 128)), _rand(n, 1, 128), v)
    np.testing.assert_allclose(out, np.broadcast_to(v.mean(0), out.shape), atol=1e-12)
    # identical keys: mean of v whatever q is
    k = np.broadcast_to(_rand(1, 1, 128), (n, 1, 128)).copy()
    out = O.attention(_rand(4, 1, 128), k, v)
    np.testing.assert_allclose(out, np.broadcast_to(v.mean(0), out.shape), atol=1e-12)
    # one dominant logit picks that value row
    k = np.zeros((n, 1, 128)); k[6, 0, 0] = 1e4
    q = np.zeros((1, 1, 128)); q[0, 0, 0] = 1.0
    np.testing.assert_allclose(O.attention(q, k, v)[0], v[6], atol=1e-12)


def test_attention_permutation_equivariance():
    q, k, v = _rand(12, 2, 128), _rand(12, 2, 128), _rand(12, 2, 128)
    perm = RNG.permutation(12)
    a = O.attention(q, k, v)
    b = O.attention(q[perm], k[perm], v[perm])
    np.testing.assert_allclose(b, a[perm], rtol=1e-12, atol=1e-13)


# --------------------------------------------------------------------------
# whole block
# --------------------------------------------------------------------------
def _tiny_weights(D, F, hd=128, norm_stress=True):
    w = {
        "wq": _rand(D, D) * 0.05, "wk": _rand(D, D) * 0.05, "wv": _rand(D, D) * 0.05,
        "wo": _rand(D, D) * 0.05, "w_gate": _rand(F, D) * 0.05, "w_up": _rand(F, D) * 0.05,
        "w_down": _rand(D, F) * 0.05,
        "q_norm": 1 + 0.1 * _rand(hd) if norm_stress else np.ones(hd),
        "k_norm": 1 + 0.1 * _rand(hd) if norm_stress else np.ones(hd),
    }
    return w


def _block_loops(x, w, segs, mod, pos, theta=O.THETA, eps=1e-6):
    """The block, one scalar at a time (independent formulation: complex
    rotations with exact angles, explicit softmax sums)."""
    N, D = len(x), len(x[0])
    F = len(w["w_gate"])
    hd = 128
    H = D // hd
    seg_of = {}
    for s, (start, count, _m) in enumerate(segs):
        for n in range(start, start + count):
            seg_of[n] = s

    def lin(W, vec):
        return [sum(W[o][i] * vec[i] for i in range(len(vec))) for o in range(len(W))]

    h = []
    for n in range(N):
        mu = sum(x[n]) / D
        var = sum((e - mu) ** 2 for e in x[n]) / D
        sh, sc, _g = mod[seg_of[n]]
        h.append([(1 + sc[i]) * (x[n][i] - mu) / math.sqrt(var + eps) + sh[i] for i in range(D)])
    q = [lin(w["wq"], hn) for hn in h]
    k = [lin(w["wk"], hn) for hn in h]
    v = [lin(w["wv"], hn) for hn in h]

    def norm_rope(vec, nw, n):
        out = list(vec)
        for hh in range(H):
            seg = vec[hh * hd:(hh + 1) * hd]
            r = math.sqrt(sum(e * e for e in seg) / hd + eps)
            seg = [seg[c] / r * nw[c] for c in range(hd)]
            for p in range(hd // 2):
                a, j = divmod(p, 16)
                z = complex(seg[2 * p], seg[2 * p + 1]) * cmath.exp(
                    1j * pos[n][a] * theta ** (-j / 16.0))
                out[hh * hd + 2 * p] = z.real
                out[hh * hd + 2 * p + 1] = z.imag
        return out

    q = [norm_rope(q[n], w["q_norm"], n) for n in range(N)]
    k = [norm_rope(k[n], w["k_norm"], n) for n in range(N)]
    o = [[0.0] * D for _ in range(N)]
    for hh in range(H):
        cols = range(hh * hd, (hh + 1) * hd)
        for i in range(N):
            logits = [sum(q[i][c] * k[j][c] for c in cols) / math.sqrt(hd) for j in range(N)]
            mx = max(logits)
            e = [math.exp(s - mx) for s in logits]
            tot = sum(e)
            for c in cols:
                o[i][c] = sum(e[j] * v[j][c] for j in range(N)) / tot
    out = []
    for n in range(N):
        a = lin(w["wo"], o[n])
        g = lin(w["w_gate"], h[n])
        u = lin(w["w_up"], h[n])
        act = [g[f] / (1 + math.exp(-g[f])) * u[f] for f in range(F)]
        m = lin(w["w_down"], act)
        gate = mod[seg_of[n]][2]
        out.append([x[n][i] + gate[i] * (a[i] + m[i]) for i in range(D)])
    return np.array(out)


def test_block_brute_force_two_heads():
    """The whole block against scalar loops on 6 tokens, 2 heads, 3 segments."""
    D, F = 256, 24
    w = _tiny_weights(D, F)
    x = _rand(6, D)
    segs = [(0, 2, 0), (2, 2, 1), (4, 2, 2)]
    mod = _rand(3, 3, D) * 0.3
    pos = O.token_positions(2, 1, 2, refs=((1, 2),))
    got = O.block_forward(x, w, segs, mod, O.rope_tables(pos))
    want = _block_loops(x.tolist(), {k_: np.asarray(v_).tolist() for k_, v_ in w.items()},
                        segs, mod.tolist(), pos.tolist())
    np.testing.assert_allclose(got, want, rtol=2e-6, atol=2e-6)


def test_block_gate_zero_is_identity():
    D, F = 128, 16
    w = _tiny_weights(D, F)
    x = _rand(5, D)
    mod = _rand(2, 3, D)
    mod[:, 2] = 0.0
    pos = O.token_positions(2, 1, 3)
    got = O.block_forward(x, w, [(0, 2, 0), (2, 3, 1)], mod, O.rope_tables(pos))
    np.testing.assert_array_equal(got, x)


def test_block_zero_projections_is_identity():
    D, F = 128, 16
    w = _tiny_weights(D, F)
    w["wo"][:] = 0
    w["w_down"][:] = 0
    x = _rand(4, D)
    pos = O.token_positions(4, 0, 0)
    got = O.block_forward(x, w, [(0, 4, 0)], _rand(1, 3, D), O.rope_tables(pos))
    np.testing.assert_array_equal(got, x)


def test_block_segment_modulation_only_touches_its_rows():
    """With the value projection zeroed, rows do not mix; changing one
    segment's modulation changes exactly that segment's rows."""
    D, F = 128, 16
    w = _tiny_weights(D, F)
    w["wv"][:] = 0
    x = _rand(7, D)
    segs = [(0, 2, 0), (2, 3, 1), (5, 2, 2)]
    mod = _rand(3, 3, D) * 0.2
    pos = O.token_positions(2, 1, 3, refs=((1, 2),))
    tab = O.rope_tables(pos)
    a = O.block_forward(x, w, segs, mod, tab)
    mod2 = mod.copy()
    mod2[1] += 0.5
    b = O.block_forward(x, w, segs, mod2, tab)
    np.testing.assert_array_equal(a[[0, 1, 5, 6]], b[[0, 1, 5, 6]])
    assert np.all(np.abs(a[2:5] - b[2:5]).max(axis=1) > 0)


def test_block_token_permutation_equivariance():
    """Permuting tokens inside a segment together with their rope rows
    permutes the output the same way."""
    D, F = 256, 16
    w = _tiny_weights(D, F)
    x = _rand(9, D)
    segs = [(0, 3, 0), (3, 6, 1)]
    mod = _rand(2, 3, D) * 0.2
    tab = O.rope_tables(O.token_positions(3, 2, 3))
    perm = np.concatenate([RNG.permutation(3), 3 + RNG.permutation(6)])
    a = O.block_forward(x, w, segs, mod, tab)
    b = O.block_forward(x[perm], w, segs, mod, tab[perm])
    np.testing.assert_allclose(b, a[perm], rtol=1e-12, atol=1e-12)


def test_block_identical_tokens_equal_one_token_block():
    """Identical input rows in one segment give identical value rows, and
    attention over equal values returns that value whatever the weights, so
    each output row is the block over that token alone -- at any position
    (the premise of the maximum-size GPU test)."""
    D, F = 256, 32
    w = _tiny_weights(D, F)
    x1 = _rand(1, D)
    mod = _rand(1, 3, D) * 0.2
    tab = O.rope_tables(O.token_positions(0, 3, 4))
    want = O.block_forward(x1, w, [(0, 1, 1)], mod, tab[5:6])
    got = O.block_forward(np.repeat(x1, 12, 0), w, [(0, 12, 1)], mod, tab)
    np.testing.assert_allclose(got, np.repeat(want, 12, 0), rtol=1e-12, atol=1e-12)
    # distinct rows do mix through attention
    x2 = np.repeat(x1, 12, 0)
    x2[7] += _rand(D)   # (a constant shift would vanish in the LayerNorm)
    got2 = O.block_forward(x2, w, [(0, 12, 1)], mod, tab)
    assert np.abs(got2[0] - want[0]).max() > 1e-6


def test_block_rows_matches_full_block():
    D, F = 256, 32
    w = _tiny_weights(D, F)
    x = _rand(11, D)
    segs = [(0, 3, 0), (3, 8, 1)]
    mod = _rand(2, 3, D) * 0.2
    tab = O.rope_tables(O.token_positions(3, 2, 4))
    full = O.block_forward(x, w, segs, mod, tab)
    rows = [0, 4, 10]
    np.testing.assert_allclose(O.block_forward_rows(x, w, segs, mod, tab, rows), full[rows],
                               rtol=1e-12, atol=1e-12)


def test_block_bf16_weight_bits_are_upcast_exactly():
    bits = synth.bf16_round_bits(np.array([1.0, -0.02, 3.1415927], np.float32))
    np.testing.assert_array_equal(O.as_float(bits, np.float64),
                                  np.array([1.0, -0.02001953125, 3.140625]))


# --------------------------------------------------------------------------
# stack
# --------------------------------------------------------------------------
def _stack_case(n_pm=2, n_joint=1):
    D, F = 128, 16
    per_mode = {m: [_tiny_weights(D, F) for _ in range(n_pm)] for m in range(3)}
    joint = [_tiny_weights(D, F) for _ in range(n_joint)]
    segs = [(0, 3, 0), (3, 4, 1), (7, 4, 2)]
    pos = O.token_positions(3, 2, 2, refs=((2, 2),))
    return D, per_mode, joint, segs, O.rope_tables(pos)


def test_stack_stage1_streams_are_independent():
    D, per_mode, _joint, segs, tab = _stack_case(n_joint=0)
    x = _rand(11, D)
    m1, m2 = _rand(3, 3, D) * 0.2, _rand(3, 3, D) * 0.2
    a = O.stack_forward(x, per_mode, [], segs, m1, m2, tab)
    x2 = x.copy()
    x2[0:3] += 1.0                      # perturb the text stream only
    b = O.stack_forward(x2, per_mode, [], segs, m1, m2, tab)
    np.testing.assert_array_equal(a[3:], b[3:])
    assert not np.allclose(a[:3], b[:3])


def test_stack_is_composition_of_blocks():
    D, per_mode, joint, segs, tab = _stack_case(n_pm=2, n_joint=2)
    x = _rand(11, D)
    m1, m2 = _rand(2, 3, 3, D) * 0.2, _rand(2, 3, 3, D) * 0.2
    got = O.stack_forward(x, per_mode, joint, segs, m1, m2, tab, per_block_mod=True)
    want = x.copy()
    for s, (start, count, mode) in enumerate(segs):
        r = slice(start, start + count)
        for b in range(2):
            want[r] = _block_loops(want[r].tolist(),
                                   {k_: np.asarray(v_).tolist() for k_, v_ in per_mode[mode][b].items()},
                                   [(0, count, mode)], m1[b][s:s + 1].tolist(),
                                   O.token_positions(3, 2, 2, refs=((2, 2),))[r].tolist())
    for b in range(2):
        want = _block_loops(want.tolist(), {k_: np.asarray(v_).tolist() for k_, v_ in joint[b].items()},
                            segs, m2[b].tolist(), O.token_positions(3, 2, 2, refs=((2, 2),)).tolist())
    np.testing.assert_allclose(got, want, rtol=1e-5, atol=1e-5)


# --------------------------------------------------------------------------
# timestep modulation and schedule
# --------------------------------------------------------------------------
def test_timestep_embedding_closed_forms():
    e0 = O.timestep_embedding(0.0)
    np.testing.assert_array_equal(e0, np.concatenate([np.ones(128), np.zeros(128)]))
    e = O.timestep_embedding(0.25)          # tau = 250
    assert e[0] == math.cos(250.0) and e[128] == math.sin(250.0)
    assert abs(e[64] - math.cos(250.0 * 10000.0 ** (-0.5))) < 1e-15


def test_modulation_text_and_reference_use_t_zero():
    """Text and reference modulation is the t = 0 path: it does not move when
    the image timestep changes, and equals a direct evaluation at t = 0."""
    D = 64
    w1, w2 = _rand(D, 256) * 0.02, _rand(D, D) * 0.02
    w_mod = {m: _rand(3 * D, D) * 0.02 for m in range(3)}
    a = O.modulation_from_t({0: 0.0, 1: 0.3, 2: 0.0}, w1, w2, w_mod)
    b = O.modulation_from_t({0: 0.0, 1: 0.9, 2: 0.0}, w1, w2, w_mod)
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[2], b[2])
    assert not np.allclose(a[1], b[1])
    # image at t = 0 with the image weights equals the text path with those weights
    c = O.modulation_from_t({1: 0.0}, w1, w2, {1: w_mod[0]})
    np.testing.assert_array_equal(c[1], a[0])
    # flow-map target embedding shifts every mode
    w1t, w2t = _rand(D, 256) * 0.02, _rand(D, D) * 0.02
    d = O.modulation_from_t({0: 0.0, 1: 0.3, 2: 0.0}, w1, w2, w_mod, t_target=0.1,
                            w1_tgt=w1t, w2_tgt=w2t)
    for m in range(3):
        assert not np.allclose(d[m], a[m])


def _golden_kv(name):
    out = {}
    for line in open(os.path.join(GOLDEN, name)):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        key, *vals = line.split()
        out[key] = [float(v) for v in vals]
    return out


def test_schedule_printed_values():
    g = _golden_kv("schedule_values.txt")
    s16 = O.shifted_sigmas(16)
    np.testing.assert_array_equal(np.round(s16[:3], 3), g["first_three"])
    np.testing.assert_array_equal(np.round(s16[13:16], 3), g["last_three"])
    assert s16[16] == g["final"][0]
    assert int((s16[:16] > 0.5).sum()) == g["steps16_above_half"][0]
    assert int((O.shifted_sigmas(50)[:50] > 0.5).sum()) == g["steps50_above_half"][0]
    assert round(s16[0] - s16[1], 3) == g["first_step_move"][0]
    assert round(s16[15] - s16[16], 3) == g["last_step_move"][0]
    assert round(O.shifted_sigmas(4)[3], 3) == g["steps4_last_nonzero"][0]
    assert round(O.shifted_sigmas(50)[9], 2) == g["steps50_sigma_at_step10"][0]


def test_euler_step_and_x0():
    x, v = _rand(4), _rand(4)
    np.testing.assert_allclose(O.euler_step(x, v, 0.8, 0.5), x - 0.3 * v)
    # integrating a constant velocity from sigma 1 to 0 lands on x - v
    s = O.shifted_sigmas(16)
    y = x.copy()
    for i in range(16):
        y = O.euler_step(y, v, s[i], s[i + 1])
    np.testing.assert_allclose(y, x - v, atol=1e-12)


# --------------------------------------------------------------------------
# the transformer call around the stack: input linears, output layer
# --------------------------------------------------------------------------
def _io_case(D=128, text_dim=96, lat=32):
    io = {"w_text": _rand(D, text_dim) * 0.05, "w_img_in": _rand(D, lat) * 0.05,
          "w_ref_in": _rand(D, lat) * 0.05, "w_final": _rand(2 * D, D) * 0.05,
          "w_out": _rand(lat, D) * 0.05}
    emb = {"w1": _rand(D, 256) * 0.05, "w2": _rand(D, D) * 0.05,
           "w1_tgt": _rand(D, 256) * 0.05, "w2_tgt": _rand(D, D) * 0.05}
    w_mod = [{m: _rand(3 * D, D) * 0.05 for m in range(3)} for _ in range(2)]
    return io, emb, w_mod


def test_input_projection_vs_torch_linear():
    io, _emb, _wm = _io_case()
    text, image, refs = _rand(3, 96), _rand(4, 32), _rand(4, 32)
    x = O.input_projection(text, image, refs, io["w_text"], io["w_img_in"], io["w_ref_in"])
    lin = torch.nn.functional.linear
    want = torch.cat([lin(torch.from_numpy(a), torch.from_numpy(io[k]))
                      for a, k in ((text, "w_text"), (image, "w_img_in"), (refs, "w_ref_in"))])
    np.testing.assert_allclose(x, want.numpy(), rtol=1e-13, atol=1e-13)
    # each token kind goes through its own matrix, in the order text, image, refs
    z = O.input_projection(text, image, refs, io["w_text"], np.zeros_like(io["w_img_in"]),
                           io["w_ref_in"])
    assert np.all(z[3:7] == 0) and np.array_equal(z[:3], x[:3]) and np.array_equal(z[7:], x[7:])


def test_output_layer_vs_torch_and_special_cases():
    io, _emb, _wm = _io_case()
    x = _rand(5, 128) * 3 + 1
    zero = np.zeros(128)
    v = O.output_layer(x, zero, zero, io["w_out"])
    xt = torch.from_numpy(x)
    ln = torch.nn.functional.layer_norm(xt, (128,), eps=1e-6)
    want = torch.nn.functional.linear(ln, torch.from_numpy(io["w_out"])).numpy()
    np.testing.assert_allclose(v, want, rtol=1e-12, atol=1e-12)
    assert v.shape == (5, 32)
    # scale = -1 removes the normalised input: every token gets shift . w_out
    shift = _rand(128)
    v = O.output_layer(x, shift, -np.ones(128), io["w_out"])
    np.testing.assert_allclose(v, np.tile(io["w_out"] @ shift, (5, 1)), rtol=1e-12, atol=1e-12)


def test_final_modulation_shares_the_embedder():
    _io, emb, w_mod = _io_case()
    # with the first two thirds of the image-mode linear, the output layer's
    # (shift, scale) equal that mode's (shift, scale)
    wf = w_mod[1][1][:256]
    for t, tt in ((0.3, None), (0.7, 0.4)):
        kw = dict(t_target=tt, w1_tgt=emb["w1_tgt"], w2_tgt=emb["w2_tgt"]) if tt is not None else {}
        got = O.final_modulation(t, emb["w1"], emb["w2"], wf, **kw)
        ref = O.modulation_from_t({1: t}, emb["w1"], emb["w2"], w_mod[1], **kw)[1]
        np.testing.assert_array_equal(got, ref[:2])
    # it follows the image timestep (unlike text and reference modulation)
    a = O.final_modulation(0.2, emb["w1"], emb["w2"], _io_case()[0]["w_final"])
    b = O.final_modulation(0.9, emb["w1"], emb["w2"], _io_case()[0]["w_final"])
    assert not np.allclose(a, b)


def _transformer_case(n_pm, n_joint):
    D, per_mode, joint, segs, tab = _stack_case(n_pm=n_pm, n_joint=n_joint)
    io, emb, w_mod = _io_case(D)
    text, image, refs = _rand(3, 96), _rand(4, 32), _rand(4, 32)
    return D, per_mode, joint, segs, tab, io, emb, w_mod, text, image, refs


def test_transformer_without_blocks_is_output_layer_of_image_inputs():
    D, per_mode, _j, segs, tab, io, emb, w_mod, text, image, refs = _transformer_case(0, 0)
    per_mode = {m: [] for m in range(3)}
    v = O.transformer_forward(text, image, refs, segs, io, emb, w_mod, per_mode, [], tab, t=0.6)
    x_img = torch.nn.functional.linear(torch.from_numpy(image), torch.from_numpy(io["w_img_in"]))
    shift, scale = O.final_modulation(0.6, emb["w1"], emb["w2"], io["w_final"])
    h = torch.nn.functional.layer_norm(x_img, (D,), eps=1e-6) * (1 + torch.from_numpy(scale)) \
        + torch.from_numpy(shift)
    want = torch.nn.functional.linear(h, torch.from_numpy(io["w_out"])).numpy()
    np.testing.assert_allclose(v, want, rtol=1e-12, atol=1e-12)


def test_transformer_stage_structure():
    D, per_mode, joint, segs, tab, io, emb, w_mod, text, image, refs = _transformer_case(1, 1)
    run = lambda tx, rf, jt: O.transformer_forward(tx, image, rf, segs, io, emb, w_mod, per_mode,
                                                   jt, tab, t=0.5, t_target=0.25)
    a = run(text, refs, [])
    # stage 1 alone: the image velocity ignores the text and the reference
    np.testing.assert_array_equal(a, run(text + 1.0, refs * 2.0, []))
    # a joint block lets both reach it
    b = run(text, refs, joint)
    assert not np.allclose(b, run(text + 1.0, refs, joint))
    assert not np.allclose(b, run(text, refs * 2.0, joint))
    assert a.shape == (4, 32)


def test_sample_loop_structure():
    """The loop calls the transformer at sigma_i (target sigma_{i+1} for the
    flow map), moves by (sigma_{i+1} - sigma_i) v, and its last x0 preview is
    the final latent (the last step lands on sigma = 0)."""
    D, per_mode, joint, segs, tab, io, emb, w_mod, text, image, refs = _transformer_case(1, 1)
    out, prev = O.sample(image, text, refs, segs, io, emb, w_mod, per_mode, joint, tab, steps=4)
    assert len(prev) == 4 and out.shape == image.shape
    np.testing.assert_allclose(prev[-1], out, rtol=1e-13, atol=1e-13)
    # step by step against explicit calls at the printed-schedule sigmas
    sig = O.shifted_sigmas(4)
    assert round(sig[3], 3) == 0.698           # "ends at 0.698 before the final jump"
    x = image.copy()
    for i in range(4):
        v = O.transformer_forward(text, x, refs, segs, io, emb, w_mod, per_mode, joint, tab,
                                  sig[i], t_target=sig[i + 1])
        np.testing.assert_array_equal(prev[i], x - sig[i] * v)
        x = x + (sig[i + 1] - sig[i]) * v
    np.testing.assert_array_equal(out, x)
    # the base model ignores the target embedder
    base, _ = O.sample(image, text, refs, segs, io, {k: emb[k] for k in ("w1", "w2")}, w_mod,
                       per_mode, joint, tab, steps=2, distilled=False)
    assert base.shape == image.shape and np.all(np.isfinite(base))


def test_transformer_text_and_reference_modulation_ignore_t():
    """Text and reference tokens are modulated at t = 0 whatever the image
    timestep [P1]: after a stack of per-mode blocks only, their rows of the
    residual stream are bit-identical for any t, while the image rows move."""
    D, per_mode, _joint, segs, tab, io, emb, w_mod, text, image, refs = _transformer_case(2, 0)
    run = lambda t: O.transformer_forward(text, image, refs, segs, io, emb, w_mod, per_mode, [],
                                          tab, t, keep=True)[1]
    a, b = run(0.2), run(0.9)
    np.testing.assert_array_equal(a[:3], b[:3])     # text rows
    np.testing.assert_array_equal(a[7:], b[7:])     # reference rows
    assert not np.allclose(a[3:7], b[3:7])          # image rows


def test_transformer_stage_modulation_goes_to_its_stage():
    """Stage-1 blocks take the stage-1 modulation linears: without joint
    blocks the stage-2 linears do not change the velocity."""
    D, per_mode, _joint, segs, tab, io, emb, w_mod, text, image, refs = _transformer_case(1, 0)
    a = O.transformer_forward(text, image, refs, segs, io, emb, w_mod, per_mode, [], tab, 0.4)
    w_mod2 = [w_mod[0], {m: w * 3.0 for m, w in w_mod[1].items()}]
    b = O.transformer_forward(text, image, refs, segs, io, emb, w_mod2, per_mode, [], tab, 0.4)
    np.testing.assert_array_equal(a, b)
    w_mod3 = [{m: w * 3.0 for m, w in w_mod[0].items()}, w_mod[1]]
    c = O.transformer_forward(text, image, refs, segs, io, emb, w_mod3, per_mode, [], tab, 0.4)
    assert not np.allclose(a, c)


# --------------------------------------------------------------------------
# rowwise FP8 (e4m3) quantisation and the block with FP8 linears
# --------------------------------------------------------------------------
def test_e4m3_format_constants():
    """The OCP e4m3 format: bias 7, 3 mantissa bits, subnormals 2^-9 apart,
    largest finite 448, the all-ones codes NaN, codes ordered by value."""
    v = O.E4M3
    assert v[0x00] == 0.0 and np.signbit(v[0x80])
    assert v[0x01] == 2.0 ** -9 and v[0x07] == 7 * 2.0 ** -9
    assert v[0x08] == 2.0 ** -6 and v[0x38] == 1.0 and v[0x39] == 1.125
    assert v[0x7E] == 448.0 and v[0x77] == 240.0
    assert np.isnan(v[0x7F]) and np.isnan(v[0xFF])
    pos = v[:0x7F]
    assert np.all(np.diff(pos) > 0)                       # monotone in the code
    np.testing.assert_array_equal(v[0x80:0xFF], -pos)     # sign-magnitude


def _e4m3_brute(y):
    """Nearest of the 127 non-negative values by search, ties to the even
    code, saturating; sign copied."""
    table = [(c, O.E4M3[c]) for c in range(0x7F)]
    out = []
    for t in np.asarray(y, np.float64).ravel():
        a = min(abs(t), 448.0)
        best = None
        for c, val in table:
            d = abs(val - a)
            if best is None or d < best[1] or (d == best[1] and c % 2 == 0):
                best = (c, d)
        out.append(best[0] | (0x80 if np.signbit(t) else 0))
    return np.array(out, np.uint8).reshape(np.shape(y))


def test_e4m3_encode_vs_brute_force():
    """Round to nearest, ties to even, on every value, every midpoint and its
    neighbours, random magnitudes over the whole range, and beyond 448."""
    vals = O.E4M3[:0x7F]
    mids = (vals[:-1] + vals[1:]) / 2
    rng = np.random.default_rng(5)
    rand = rng.standard_normal(3000) * np.exp2(rng.uniform(-12, 10, 3000))
    y = np.concatenate([vals, -vals, mids, -mids, np.nextafter(mids, 0), np.nextafter(mids, 1e9),
                        rand, [448.0, 449.0, 463.9, 464.0, 465.0, 1e6, -1e6, 2.0 ** -10,
                               1.5 * 2.0 ** -10, -2.0 ** -11, 0.0, -0.0]])
    y = y.astype(np.float32).astype(np.float64)            # the inputs are fp32
    np.testing.assert_array_equal(O.e4m3_encode(y), _e4m3_brute(y))


def test_e4m3_ties_go_to_even_codes():
    vals = O.E4M3[:0x7F]
    mids = (vals[:-1] + vals[1:]) / 2
    codes = O.e4m3_encode(mids)
    assert np.all(codes % 2 == 0)
    assert np.all((codes == np.arange(0x7E)) | (codes == np.arange(1, 0x7F)))


def test_quantize_rowwise_scale_and_error_bound():
    """Scale = row max / 448; the row maximum maps to +-448; every element
    within half a step of its value (2^-4 relative for normals, 2^-10 s in
    the subnormal range)."""
    rng = np.random.default_rng(6)
    a = (rng.standard_normal((40, 300)) * np.exp2(rng.uniform(-20, 20, (40, 1)))).astype(np.float32)
    codes, s = O.quantize_rowwise(a)
    amax = np.abs(a).max(axis=1)
    np.testing.assert_array_equal(s, (amax / np.float32(448)).astype(np.float32))
    arg = np.abs(a).argmax(axis=1)
    assert np.all(np.abs(O.E4M3[codes[np.arange(40), arg]]) == 448.0)
    deq = O.dequantize_rowwise(codes, s)
    y = np.abs(a.astype(np.float64)) / s[:, None].astype(np.float64)   # position on the grid
    err = np.abs(deq - a) / s[:, None]
    bound = np.where(y >= 2.0 ** -6, y * 2.0 ** -4, 2.0 ** -10) * (1 + 1e-6)
    assert np.all(err <= bound)
    assert np.all(np.sign(deq) * np.sign(a) >= 0)


def test_quantize_rowwise_special_rows():
    """A zero row gives scale 0 and zero codes; a row already on the e4m3
    grid with maximum 448 is returned as is (scale 1); scaling a row by a
    power of two scales only its scale."""
    rng = np.random.default_rng(7)
    on_grid = O.E4M3[rng.integers(0, 0x7E, (3, 64))] * rng.choice([-1, 1], (3, 64))
    on_grid[:, 5] = 448.0
    rows = np.vstack([np.zeros((1, 64)), on_grid])
    codes, s = O.quantize_rowwise(rows)
    assert s[0] == 0 and np.all(O.E4M3[codes[0]] == 0)
    np.testing.assert_array_equal(s[1:], 1.0)
    np.testing.assert_array_equal(O.E4M3[codes[1:]], on_grid)
    b = rng.standard_normal((4, 50)).astype(np.float32)
    c1, s1 = O.quantize_rowwise(b)
    c2, s2 = O.quantize_rowwise(b * np.float32(2.0 ** -7))
    np.testing.assert_array_equal(c1, c2)
    np.testing.assert_array_equal(s2, s1 * np.float32(2.0 ** -7))


def test_fused_matrices_split_back_into_the_linears():
    D, F = 128, 48
    w = _tiny_weights(D, F)
    w1, w2 = O.fused_block_matrices(w)
    assert w1.shape == (3 * D + 2 * F, D) and w2.shape == (D, D + F)
    h = _rand(5, D)
    y = h @ w1.T
    for name, lo, hi in [("wq", 0, D), ("wk", D, 2 * D), ("wv", 2 * D, 3 * D),
                         ("w_gate", 3 * D, 3 * D + F), ("w_up", 3 * D + F, 3 * D + 2 * F)]:
        np.testing.assert_allclose(y[:, lo:hi], h @ w[name].T, rtol=1e-12, atol=1e-12)
    o, act = _rand(5, D), _rand(5, F)
    np.testing.assert_allclose(np.hstack([o, act]) @ w2.T, o @ w["wo"].T + act @ w["w_down"].T,
                               rtol=1e-12, atol=1e-12)


def _fp8_case(D=256, F=64, n=9):
    w = _tiny_weights(D, F)
    x = _rand(n, D)
    segs = [(0, 3, 0), (3, n - 3, 1)]
    mod = _rand(2, 3, D) * 0.2
    tab = O.rope_tables(O.token_positions(3, 2, (n - 3) // 2))
    return w, x, segs, mod, tab


def test_quantized_block_with_identity_quantiser_is_the_block():
    """With the unquantised fused weights and no activation quantisation the
    FP8 block's structure reduces to block_forward (pinned by brute force)."""
    w, x, segs, mod, tab = _fp8_case()
    w1, w2 = O.fused_block_matrices(w)
    got = O.block_forward_quantized(x, w1, w2, (w["q_norm"], w["k_norm"]), segs, mod, tab,
                                    lambda a: a)
    np.testing.assert_allclose(got, O.block_forward(x, w, segs, mod, tab), rtol=1e-12, atol=1e-12)
    rows = [0, 4, 8]
    got_r = O.block_forward_quantized(x, w1, w2, (w["q_norm"], w["k_norm"]), segs, mod, tab,
                                      lambda a: a, rows=rows)
    np.testing.assert_allclose(got_r, got[rows], rtol=1e-12, atol=1e-12)


def test_quantized_block_quantises_h_then_the_concatenation():
    """The activation quantiser sees exactly the two GEMM inputs: the
    modulated h [n][D], then [o | act] [n][D + F]."""
    w, x, segs, mod, tab = _fp8_case()
    _, inter = O.block_forward(x, w, segs, mod, tab, keep=True)
    seen = []

    def record(a):
        seen.append(np.array(a))
        return a

    w1, w2 = O.fused_block_matrices(w)
    O.block_forward_quantized(x, w1, w2, (w["q_norm"], w["k_norm"]), segs, mod, tab, record)
    assert len(seen) == 2
    np.testing.assert_allclose(seen[0], inter["h"], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(seen[1], np.hstack([inter["o"], inter["act"]]), rtol=1e-10,
                               atol=1e-12)


def test_fp8_block_is_the_block_on_dequantised_operands():
    """block_forward_fp8 uses the dequantised codes of quantize_block_weights
    and rowwise-quantised activations; its change against the bf16-weight
    block is of the size 3-bit mantissas give (a few percent of the block
    delta), and is not zero."""
    w, x, segs, mod, tab = _fp8_case(n=13)
    w8 = O.quantize_block_weights(w)
    w1, w2 = O.fused_block_matrices(w)
    c1, s1 = w8["w1"]
    c1_want, s1_want = O.quantize_rowwise(w1)
    np.testing.assert_array_equal(c1, c1_want)
    np.testing.assert_array_equal(s1, s1_want)
    got = O.block_forward_fp8(x, w8, segs, mod, tab)
    ref = O.block_forward(x, w, segs, mod, tab)
    d_got, d_ref = got - x, ref - x
    rel = np.linalg.norm(d_got - d_ref) / np.linalg.norm(d_ref)
    assert 1e-3 < rel < 0.1, rel
    deq = O.block_forward_quantized(x, O.dequantize_rowwise(*w8["w1"]),
                                    O.dequantize_rowwise(*w8["w2"]),
                                    (w["q_norm"], w["k_norm"]), segs, mod, tab,
                                    O.fake_quantize_rows)
    np.testing.assert_array_equal(got, deq)
    rows = [1, 6, 12]
    np.testing.assert_allclose(O.block_forward_fp8(x, w8, segs, mod, tab, rows=rows), got[rows],
                               rtol=1e-12, atol=1e-12)


def test_quantize_rowwise_decides_in_fp32():
    """The rounding decision is taken on the fp32 product v * (448 / a): rows
    built so that this product lands exactly on e4m3 midpoints while the
    exact product does not must round to the even neighbour of the
    midpoint (brute-force search on the fp32 product)."""
    mids = (O.E4M3[1:0x7E] + O.E4M3[2:0x7F]) / 2
    rows, discriminating = [], 0
    for amax in (1344.0, 2240.0, 3136.0, 492.8, 1000.0):
        mult = np.float32(448.0) / np.float32(amax)
        row = [np.float32(amax)]
        for mdp in mids[::3]:
            x = np.float32(mdp / float(mult))
            for _ in range(8):          # walk to an x whose fp32 product is the midpoint
                p = np.float32(x * mult)
                if p == mdp:
                    break
                x = np.nextafter(x, np.float32(np.inf) if p < mdp else np.float32(-np.inf))
            if np.float32(x * mult) == mdp and 0 < x < amax:
                row.append(x)
                discriminating += float(x) * float(mult) != mdp
        rows.append(np.array(row + [0.0] * (64 - len(row)), np.float32)[:64])
    a = np.stack(rows)
    assert discriminating > 10       # the exact products miss the midpoints
    codes, _ = O.quantize_rowwise(a)
    amax = np.abs(a).max(axis=1)
    prod = (a * (np.float32(448.0) / amax)[:, None]).astype(np.float32)
    np.testing.assert_array_equal(codes, _e4m3_brute(prod.astype(np.float64)))
