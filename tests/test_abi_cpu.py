"""Host-side checks of the C ABI that need no GPU: the library loads, exports
every function include/flux3.h declares, sizes its workspace as documented,
and rejects bad arguments with the documented status before any HIP call.

Only failing calls are made here (validation runs before anything is
enqueued); no valid compute call is issued without a GPU.
"""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

import latent_flow_matching_flux_amd as F
from latent_flow_matching_flux_amd import _lib as L
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "flux3.h")

OK, E_INVALID, E_SHAPE, E_UNSUPPORTED, E_ALIGN, E_WORKSPACE = 0, -1, -2, -3, -4, -5
FAKE = 0x7F0000000000          # a 256-byte aligned address that is never dereferenced


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(flux3_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    lib = F.load()
    declared = header_functions()
    assert declared == sorted(L.EXPORTS)
    for name in declared:
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", F.LIB_PATH], capture_output=True,
                         text=True).stdout
    exported = set(re.findall(r" T (flux3_\w+)", out))
    assert set(declared) <= exported


def _dims(width=3072, heads=24, head_dim=128, hidden=9216):
    return L.Dims(width, heads, head_dim, hidden)


def _w(addr=FAKE):
    return L.BlockWeights(*[addr + 4096 * i for i in range(9)])


def _call_block(dims=None, w=None, x=FAKE, n=336, segs=((0, 80, 0), (80, 256, 1)),
                mod=FAKE, rope=FAKE, ws=FAKE, ws_bytes=None):
    lib = F.load()
    d = dims if dims is not None else _dims()
    seg_arr, n_segs = L.make_segments(list(segs))
    if ws_bytes is None:
        ws_bytes = lib.flux3_workspace_bytes(ctypes.byref(d), n) if d.head_dim == 128 else 1 << 30
    wp = ctypes.byref(w if w is not None else _w())
    return lib.flux3_block_forward(ctypes.byref(d), wp, x, n, seg_arr, n_segs, mod, rope, ws,
                                   ws_bytes, 0)


def test_workspace_bytes_formula():
    d = synth.DIMS
    per_tok = (d.width + 3 * d.width + d.width + d.mlp_hidden) * 2   # h, q, k, vt, cat in bf16
    part = 2 * 256 * 256 * 256 * 4        # two fp32 256x256 partial tiles per stream-K group
    for n in (1, 7, 256, 336, 8432, 65776):
        n_pad = (n + 255) // 256 * 256
        assert F.workspace_bytes(d, n) == n_pad * per_tok + part
    assert F.workspace_bytes(synth.Dims(3072, 24, 64, 9216), 10) == 0
    lay = F.workspace_layout(d, 8432)
    assert lay.n_pad == 8448 and lay.total == F.workspace_bytes(d, 8432)
    assert lay.h == 0 and lay.q < lay.k < lay.vt < lay.cat < lay.part < lay.total
    assert lay.total - lay.part == part
    assert all(off % 256 == 0 for off in (lay.q, lay.k, lay.vt, lay.cat, lay.part))


def test_layout_tokens():
    for wl in synth.WORKLOADS.values():
        assert F.layout_tokens(wl.layout) == wl.n_tokens
    assert F.layout_tokens(synth.RopeLayout(-1, 2, 2)) == -1
    assert F.layout_tokens(synth.RopeLayout(0, 2, 0)) == -1
    assert F.layout_tokens(synth.RopeLayout(0, 1, 1, tuple((1, 1) for _ in range(16)))) == -1


@pytest.mark.parametrize("dims,status", [
    (_dims(head_dim=64), E_UNSUPPORTED),
    (_dims(width=3072, heads=23), E_UNSUPPORTED),
    (_dims(width=3000), E_UNSUPPORTED),
    (_dims(hidden=9200), E_UNSUPPORTED),
    (_dims(hidden=0), E_UNSUPPORTED),
    (_dims(width=514 * 128, heads=514), E_UNSUPPORTED),
    (_dims(width=2 ** 30, heads=2 ** 23), E_UNSUPPORTED),
    (_dims(hidden=(1 << 18) + 128), E_UNSUPPORTED),
    (_dims(hidden=2 ** 31 - 128), E_UNSUPPORTED),
])
def test_block_rejects_unsupported_dims(dims, status):
    assert _call_block(dims=dims) == status


def test_block_rejects_null_and_misaligned():
    assert F.load().flux3_block_forward(None, ctypes.byref(_w()), FAKE, 336, None, 0, FAKE, FAKE,
                                        FAKE, 1 << 40, 0) == E_INVALID
    assert _call_block(x=None) == E_INVALID
    assert _call_block(mod=None) == E_INVALID
    assert _call_block(rope=None) == E_INVALID
    w = _w()
    w.w_down = None
    assert _call_block(w=w) == E_INVALID
    assert b"w_down" in F.load().flux3_last_error_detail()
    assert _call_block(x=FAKE + 4) == E_ALIGN
    w = _w()
    w.wk = FAKE + 2
    assert _call_block(w=w) == E_ALIGN
    assert _call_block(ws=FAKE + 16) == E_ALIGN


def test_block_rejects_bad_segments():
    assert _call_block(segs=()) == E_SHAPE                                  # no segments
    assert _call_block(segs=((0, 80, 0), (80, 255, 1))) == E_SHAPE         # short
    assert _call_block(segs=((0, 80, 0), (81, 255, 1))) == E_SHAPE         # gap
    assert _call_block(segs=((0, 80, 1), (80, 256, 0))) == E_SHAPE         # order
    assert _call_block(segs=((0, 80, 0), (80, 256, 3))) == E_INVALID       # mode
    assert _call_block(segs=((0, 0, 0), (0, 336, 1))) == E_SHAPE          # empty
    assert _call_block(segs=tuple((i, 1, 0) for i in range(17)), n=17) == E_SHAPE


def test_block_sizes_and_workspace():
    assert _call_block(n=-1) == E_SHAPE
    assert _call_block(n=(1 << 20) + 1, segs=((0, (1 << 20) + 1, 0),)) == E_SHAPE
    assert _call_block(ws=None) == E_WORKSPACE
    need = F.workspace_bytes(synth.DIMS, 336)
    assert _call_block(ws_bytes=need - 1) == E_WORKSPACE
    # empty call is a no-op
    assert _call_block(n=0, segs=()) == OK
    assert _call_block(n=0, segs=((0, 1, 0),)) == E_SHAPE


def test_block_noalloc_validation():
    """The allocation-free block validates like flux3_block_forward and
    rejects sizes beyond its array before touching a device."""
    lib = F.load()
    d = _dims()
    seg_arr, n_segs = L.make_segments([(0, 80, 0), (80, 256, 1)])
    def call(n=336, segs=(seg_arr, n_segs), x=FAKE, w=None):
        return lib.flux3_block_forward_noalloc(ctypes.byref(d), ctypes.byref(w or _w()), x, n,
                                               segs[0], segs[1], FAKE, FAKE, 0)
    assert call(x=None) == E_INVALID
    assert call(x=FAKE + 4) == E_ALIGN
    assert call(n=337) == E_SHAPE
    big = L.make_segments([(0, 1025, 0)])
    assert call(n=1025, segs=big) == E_WORKSPACE
    assert b"1025" in lib.flux3_last_error_detail()
    assert call(n=0, segs=L.make_segments([])) == OK
    # the array holds exactly the 1024-token intermediates at the model dims
    assert F.workspace_layout(synth.DIMS, 1024).part == L.NOALLOC_SCRATCH_BYTES
    assert F.workspace_layout(synth.DIMS, 1025).part > L.NOALLOC_SCRATCH_BYTES


def test_rope_build_validation():
    lib = F.load()
    lay = L.make_layout(synth.workload("block336").layout)
    assert lib.flux3_rope_tables_build(None, FAKE, 336, 0) == E_INVALID
    assert lib.flux3_rope_tables_build(ctypes.byref(lay), FAKE, 335, 0) == E_SHAPE
    assert lib.flux3_rope_tables_build(ctypes.byref(lay), None, 336, 0) == E_INVALID
    assert lib.flux3_rope_tables_build(ctypes.byref(lay), FAKE + 8, 336, 0) == E_ALIGN
    many = L.make_layout(synth.RopeLayout(0, 1, 1, tuple((1, 1) for _ in range(16))))
    assert lib.flux3_rope_tables_build(ctypes.byref(many), FAKE, 17, 0) == E_SHAPE
    empty = L.make_layout(synth.RopeLayout(0, 0, 0))
    assert lib.flux3_rope_tables_build(ctypes.byref(empty), None, 0, 0) == OK


def _call_stack(n_pm=5, n_joint=28, per_mode=True, joint=True, m1=FAKE, m2=FAKE, stride=0,
                segs=((0, 80, 0), (80, 256, 1)), ws_bytes=None):
    lib = F.load()
    d = _dims()
    pm = (L.BlockWeights * (3 * max(n_pm, 1)))(*[_w() for _ in range(3 * max(n_pm, 1))])
    jt = (L.BlockWeights * max(n_joint, 1))(*[_w() for _ in range(max(n_joint, 1))])
    seg_arr, n_segs = L.make_segments(list(segs))
    n = sum(s[1] for s in segs)
    if ws_bytes is None:
        ws_bytes = lib.flux3_workspace_bytes(ctypes.byref(d), n)
    return lib.flux3_stack_forward(ctypes.byref(d), pm if per_mode else None, n_pm,
                                   jt if joint else None, n_joint, FAKE, n, seg_arr, n_segs,
                                   m1, m2, stride, FAKE, FAKE, ws_bytes, 0)


def test_stack_validation():
    assert _call_stack(per_mode=False) == E_INVALID
    assert _call_stack(joint=False) == E_INVALID
    assert _call_stack(m1=None) == E_INVALID
    assert _call_stack(m2=None) == E_INVALID
    assert _call_stack(m2=FAKE + 4) == E_ALIGN
    assert _call_stack(stride=-4) == E_SHAPE
    assert _call_stack(stride=6) == E_ALIGN
    assert _call_stack(n_pm=-1) == E_SHAPE
    assert _call_stack(ws_bytes=100) == E_WORKSPACE
    assert _call_stack(segs=((0, 80, 2), (80, 256, 1))) == E_SHAPE


def test_status_strings():
    for s in (0, -1, -2, -3, -4, -5, -6):
        assert F.status_string(s) and F.status_string(s) != "unknown status"
    assert F.status_string(-99) == "unknown status"


def test_binding_has_no_cpu_fallback(tmp_path):
    """Loading from a path without the library raises instead of falling back."""
    saved = L._lib
    L._lib = None
    try:
        with pytest.raises(ImportError):
            L.load(str(tmp_path / "missing.so"))
    finally:
        L._lib = saved


def test_packed_layout_reader():
    from layouts import unpack_rows, pack_rows_loops
    rng = np.random.default_rng(0)
    for R, K in ((8, 64), (16, 128), (24, 192)):
        x = rng.standard_normal((R, K)).astype(np.float32)
        p = pack_rows_loops(x)
        # every 1-KiB block (512 bf16 values) holds 8 whole rows of 64 k-values
        blk = p.reshape(-1, 512)
        assert blk.shape[0] == (R // 8) * (K // 64)
        assert np.array_equal(np.sort(blk[0]), np.sort(x[:8, :64].ravel()))
        assert np.array_equal(unpack_rows(p, R, K), x)


def test_packed_fp8_layout_reader():
    """The fp8 code layout read back two ways: by its own definition and as
    the bytes of the bf16 layout of code pairs."""
    from layouts import unpack8_rows, pack8_rows_loops
    rng = np.random.default_rng(1)
    for R, K in ((8, 128), (16, 256), (24, 384)):
        x = rng.integers(0, 256, (R, K)).astype(np.uint8)
        p = pack8_rows_loops(x)
        blk = p.reshape(-1, 1024)
        assert blk.shape[0] == (R // 8) * (K // 128)
        assert np.array_equal(np.sort(blk[0]), np.sort(x[:8, :128].ravel()))
        assert np.array_equal(unpack8_rows(p, R, K), x)


def test_modulation_workspace_and_validation():
    d = _dims()
    assert F.modulation_workspace_bytes(synth.DIMS) == (4 * 256 + 8 * 3072) * 4
    assert F.modulation_workspace_bytes(synth.Dims(3072, 24, 64, 9216)) == 0
    lib = F.load()
    segs = [(0, 240, 0), (240, 4096, 1), (4336, 4096, 2)]
    seg_arr, n_segs = L.make_segments(segs)
    ws_bytes = F.modulation_workspace_bytes(synth.DIMS)

    def call(w=None, t=(0.0, 0.5, 0.0), t_target=-1.0, dims=None, mod=FAKE, ws=FAKE,
             nbytes=ws_bytes):
        W = w if w is not None else L.ModulationWeights(FAKE, FAKE, None, None,
                                                        (ctypes.c_void_p * 3)(FAKE, FAKE, FAKE))
        tt = (ctypes.c_float * 3)(*t) if t is not None else None
        return lib.flux3_modulation_forward(ctypes.byref(dims or d), ctypes.byref(W), tt,
                                            t_target, seg_arr, n_segs, mod, ws, nbytes, 0)

    assert call(t=None) == E_INVALID
    assert call(t=(0.0, float("nan"), 0.0)) == E_INVALID
    assert call(t_target=float("nan")) == E_INVALID
    assert call(t_target=0.1) == E_INVALID            # target embedder missing
    no_ref = L.ModulationWeights(FAKE, FAKE, None, None, (ctypes.c_void_p * 3)(FAKE, FAKE, None))
    assert call(w=no_ref) == E_INVALID                # a segment uses mode 2
    assert call(dims=_dims(width=5120, heads=40, hidden=15360)) == E_UNSUPPORTED
    assert call(nbytes=ws_bytes - 4) == E_WORKSPACE
    assert call(mod=FAKE + 4) == E_ALIGN
    assert call(ws=FAKE + 16) == E_ALIGN


def test_weights_pack_sizes_and_validation():
    lib = F.load()
    d = _dims()
    D, Fh = 3072, 9216
    assert F.weights_packed_bytes(synth.DIMS) == 2 * (4 * D * D + 3 * D * Fh) == 245366784
    assert lib.flux3_weights_packed_bytes(ctypes.byref(_dims(head_dim=64))) == 0
    need = F.weights_packed_bytes(synth.DIMS)
    out = L.BlockWeights()

    def pack(w=None, buf=FAKE + (1 << 32), nbytes=need, o=out, dims=d):
        return lib.flux3_weights_pack(ctypes.byref(dims), None if w is False else
                                      ctypes.byref(w if w is not None else _w()), buf, nbytes,
                                      None if o is None else ctypes.byref(o), 0)

    assert pack(w=False) == E_INVALID                     # no input struct
    packed = _w()
    packed.layout = L.WEIGHTS_PACKED
    assert pack(w=packed) == E_INVALID                    # already packed
    assert b"already packed" in lib.flux3_last_error_detail()
    assert pack(o=None) == E_INVALID
    assert pack(buf=None) == E_WORKSPACE
    assert pack(buf=FAKE + 16) == E_ALIGN
    assert pack(nbytes=need - 1) == E_WORKSPACE
    assert pack(dims=_dims(width=3000)) == E_UNSUPPORTED
    w = _w()
    w.w_up = FAKE + 8
    assert pack(w=w) == E_ALIGN
    # a block call rejects an unknown layout value before anything runs
    bad = _w()
    bad.layout = 7
    assert _call_block(w=bad) == E_INVALID
    assert b"layout" in lib.flux3_last_error_detail()


def test_weights_fp8r_sizes_and_validation():
    lib = F.load()
    d = _dims()
    D, Fh = 3072, 9216
    # one byte per code, scales fp32, each piece 256-byte aligned
    assert F.weights_fp8r_bytes(synth.DIMS) == \
        4 * D * D + 3 * D * Fh + 4 * (3 * D + 2 * Fh) + 4 * D == 122806272
    assert lib.flux3_weights_fp8r_bytes(ctypes.byref(_dims(head_dim=64))) == 0
    need = F.weights_fp8r_bytes(synth.DIMS)
    out = L.BlockWeights()

    def quant(w=None, buf=FAKE + (1 << 32), nbytes=need, o=out, dims=d):
        return lib.flux3_weights_quantize_fp8r(ctypes.byref(dims), None if w is False else
                                               ctypes.byref(w if w is not None else _w()), buf,
                                               nbytes, None if o is None else ctypes.byref(o), 0)

    assert quant(w=False) == E_INVALID
    packed = _w()
    packed.layout = L.WEIGHTS_PACKED
    assert quant(w=packed) == E_INVALID
    assert b"Linear" in lib.flux3_last_error_detail()
    assert quant(o=None) == E_INVALID
    assert quant(buf=None) == E_WORKSPACE
    assert quant(buf=FAKE + 16) == E_ALIGN
    assert quant(nbytes=need - 1) == E_WORKSPACE
    assert quant(dims=_dims(width=3000)) == E_UNSUPPORTED
    # the per-token quantiser's row limit and the workspace room for [o | act]
    assert quant(dims=_dims(hidden=13568)) == E_UNSUPPORTED
    assert b"16384" in lib.flux3_last_error_detail()
    assert quant(dims=_dims(width=256, heads=2, hidden=7 * 256)) == E_UNSUPPORTED
    # a block call with fp8r weights needs both scale arrays, aligned
    w8 = _w()
    w8.layout = L.WEIGHTS_FP8R
    assert _call_block(w=w8) == E_INVALID
    assert b"s_proj" in lib.flux3_last_error_detail()
    w8.s_proj = FAKE + (1 << 33)
    w8.s_out = FAKE + (1 << 33) + 8
    assert _call_block(w=w8) == E_ALIGN
    w8.s_out = FAKE + (1 << 33) + 65536
    small = _dims(width=256, heads=2, hidden=7 * 256)
    assert _call_block(dims=small, w=w8) == E_UNSUPPORTED


def test_transformer_workspace_and_validation():
    lib = F.load()
    d = _dims()
    io_dims = L.IoDims(20480, 128)
    n = 336
    need = F.transformer_workspace_bytes(synth.DIMS, io_dims, n)
    assert need >= F.workspace_bytes(synth.DIMS, n) + n * 3072 * 4
    for bad in (L.IoDims(20480, 100), L.IoDims(20480, 512), L.IoDims(100, 128),
                L.IoDims((1 << 18) + 64, 128), L.IoDims(2 ** 31 - 64, 128)):
        assert F.transformer_workspace_bytes(synth.DIMS, bad, n) == 0
    io = L.IoWeights(*[FAKE + 4096 * i for i in range(5)])
    mw = (L.ModulationWeights * 2)()
    for k in range(2):
        mw[k].w1, mw[k].w2 = FAKE, FAKE + 256
        for m in range(3):
            mw[k].w_mod[m] = FAKE + 512 * (m + 1)
    pm = (L.BlockWeights * 3)(_w(), _w(), _w())
    jt = (L.BlockWeights * 1)(_w())
    segs3 = ((0, 80, 0), (80, 128, 1), (208, 128, 2))

    def call(dims=d, iod=io_dims, iow=io, m=mw, text=FAKE, image=FAKE, refs=FAKE,
             segs=segs3, t=0.5, tt=-1.0, rope=FAKE, vel=FAKE, ws=FAKE, ws_bytes=None):
        seg_arr, n_segs = L.make_segments(list(segs))
        nn = sum(c for _s, c, _m in segs)
        if ws_bytes is None:
            ws_bytes = F.transformer_workspace_bytes(synth.DIMS, io_dims, nn)
        return lib.flux3_transformer_forward(
            ctypes.byref(dims), None if iod is None else ctypes.byref(iod),
            None if iow is None else ctypes.byref(iow), m, pm, 1, jt, 1, text, image, refs,
            seg_arr, n_segs, t, tt, rope, vel, ws, ws_bytes, 0)

    assert call(iod=None) == E_INVALID
    assert call(iod=L.IoDims(20480, 96)) == E_UNSUPPORTED
    assert call(iod=L.IoDims((1 << 18) + 64, 128)) == E_UNSUPPORTED
    assert call(iow=None) == E_INVALID
    assert call(m=None) == E_INVALID
    assert call(segs=((0, 80, 0), (80, 128, 2))) == E_SHAPE                 # no image
    assert call(segs=((0, 80, 0), (80, 64, 1), (144, 64, 1))) == E_SHAPE    # two images
    assert call(image=None) == E_INVALID
    assert call(text=None) == E_INVALID                                      # text segment present
    assert call(refs=FAKE + 8) == E_ALIGN
    assert call(vel=None) == E_INVALID
    assert call(t=float("nan")) == E_INVALID
    assert call(tt=float("nan")) == E_INVALID
    assert call(tt=0.25) == E_INVALID                                        # no target embedder
    assert call(ws=None) == E_WORKSPACE
    assert call(ws_bytes=1 << 20) == E_WORKSPACE
    w_final_null = L.IoWeights(FAKE, FAKE, FAKE, None, FAKE)
    assert call(iow=w_final_null) == E_INVALID
    assert b"w_final" in lib.flux3_last_error_detail()
    # text and references are optional when no segment holds them
    no_ref = L.IoWeights(FAKE, FAKE, None, FAKE, FAKE)
    assert call(iow=no_ref, refs=None, segs=((0, 80, 0), (80, 128, 1)), ws=None) == E_WORKSPACE


def test_sigmas_schedule_and_validation():
    from oracle import flux3_oracle as O
    for steps in (1, 4, 16, 50):
        got = np.array(F.sigmas(steps), np.float32)
        want = O.shifted_sigmas(steps).astype(np.float32)
        assert got.shape == want.shape and got[-1] == 0.0
        np.testing.assert_array_max_ulp(got, want, maxulp=1)
    s16 = F.sigmas(16)
    assert [round(v, 3) for v in s16[:3]] == [1.0, 0.99, 0.98]
    assert [round(v, 3) for v in s16[13:16]] == [0.615, 0.497, 0.316]
    lib = F.load()
    buf = (ctypes.c_float * 4)()
    assert lib.flux3_sigmas(0, 6.93, buf) == E_SHAPE
    assert lib.flux3_sigmas(3, 0.0, buf) == E_INVALID
    assert lib.flux3_sigmas(3, float("nan"), buf) == E_INVALID
    assert lib.flux3_sigmas(3, 6.93, None) == E_INVALID


def test_euler_and_sample_validation():
    lib = F.load()
    assert lib.flux3_euler_step(None, FAKE, None, 128, 1.0, 0.9, 0) == E_INVALID
    assert lib.flux3_euler_step(FAKE, FAKE, None, 126, 1.0, 0.9, 0) == E_SHAPE
    assert lib.flux3_euler_step(FAKE, FAKE + 4, None, 128, 1.0, 0.9, 0) == E_ALIGN
    assert lib.flux3_euler_step(FAKE, FAKE, None, 128, float("inf"), 0.9, 0) == E_INVALID
    io_dims = L.IoDims(20480, 128)
    need = F.sample_workspace_bytes(synth.DIMS, io_dims, 336)
    assert need >= F.transformer_workspace_bytes(synth.DIMS, io_dims, 336) + 336 * 128 * 4
    seg_arr, n_segs = L.make_segments([(0, 80, 0), (80, 256, 1)])
    io = L.IoWeights(*[FAKE + 4096 * i for i in range(5)])
    mw = (L.ModulationWeights * 2)()
    args = lambda steps, ws, nbytes: (ctypes.byref(_dims()), ctypes.byref(io_dims),
                                      ctypes.byref(io), mw, None, 0, None, 0, FAKE, FAKE, None,
                                      seg_arr, n_segs, steps, 6.93, 1, FAKE, None, ws, nbytes, 0)
    assert lib.flux3_sample(*args(0, FAKE, need)) == E_SHAPE
    assert lib.flux3_sample(*args(16, FAKE, need - 1)) == E_WORKSPACE
    assert lib.flux3_sample(*args(16, None, need)) == E_WORKSPACE
    # reaches the transformer call's own checks (no modulation weights)
    assert lib.flux3_sample(*args(16, FAKE, need)) == E_INVALID
