"""ctypes binding to libflux3.so: argument marshalling only.

Every function here converts Python/torch arguments to the C ABI declared in
include/flux3.h and calls it; all computation runs in the library's HIP
kernels.  torch is used for device memory and streams.  If the library is
missing the import-time loader raises: there is no fallback path.
"""
import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
# FLUX3_LIB names another build of the library (the sanitizer check uses it)
LIB_PATH = os.environ.get("FLUX3_LIB") or os.path.join(HERE, "libflux3.so")

FLUX3_OK = 0
STATUS_NAMES = {0: "FLUX3_OK", -1: "FLUX3_E_INVALID", -2: "FLUX3_E_SHAPE",
                -3: "FLUX3_E_UNSUPPORTED", -4: "FLUX3_E_ALIGN",
                -5: "FLUX3_E_WORKSPACE", -6: "FLUX3_E_HIP"}
MAX_SEGMENTS = 16
MAX_REFS = 15
NOALLOC_SCRATCH_BYTES = 48 * 1024 * 1024   # FLUX3_NOALLOC_SCRATCH_BYTES

# exported symbols, in the order include/flux3.h declares them
EXPORTS = ("flux3_layout_tokens", "flux3_rope_tables_build", "flux3_workspace_bytes",
           "flux3_workspace_layout_get", "flux3_block_forward", "flux3_block_forward_noalloc",
           "flux3_stack_forward",
           "flux3_weights_packed_bytes", "flux3_weights_pack",
           "flux3_weights_fp8r_bytes", "flux3_weights_quantize_fp8r",
           "flux3_transformer_workspace_bytes", "flux3_transformer_forward",
           "flux3_sigmas", "flux3_euler_step", "flux3_sample_workspace_bytes", "flux3_sample",
           "flux3_modulation_workspace_bytes", "flux3_modulation_forward",
           "flux3_profile_enable", "flux3_profile_reset", "flux3_profile_read",
           "flux3_profile_read_tokens",
           "flux3_device_query", "flux3_set_debug_sync", "flux3_status_string",
           "flux3_last_error_detail")
KERNELS = ("rope_tables", "ln_modulate", "gemm_proj", "attention", "gemm_out", "modulation",
           "io_linears", "euler", "quant")


class Flux3Error(RuntimeError):
    def __init__(self, status, detail):
        self.status = status
        self.detail = detail
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {detail}")


class Dims(ctypes.Structure):
    _fields_ = [("width", ctypes.c_int32), ("heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("mlp_hidden", ctypes.c_int32)]


class Segment(ctypes.Structure):
    _fields_ = [("start", ctypes.c_int32), ("count", ctypes.c_int32), ("mode", ctypes.c_int32)]


WEIGHTS_LINEAR, WEIGHTS_PACKED, WEIGHTS_FP8R = 0, 1, 2
MATRICES = ("wq", "wk", "wv", "wo", "w_gate", "w_up", "w_down")


class BlockWeights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in MATRICES + ("q_norm", "k_norm")] + \
               [("layout", ctypes.c_int32), ("s_proj", ctypes.c_void_p),
                ("s_out", ctypes.c_void_p)]


class ModulationWeights(ctypes.Structure):
    _fields_ = [("w1", ctypes.c_void_p), ("w2", ctypes.c_void_p), ("w1_tgt", ctypes.c_void_p),
                ("w2_tgt", ctypes.c_void_p), ("w_mod", ctypes.c_void_p * 3)]


class IoDims(ctypes.Structure):
    _fields_ = [("text_dim", ctypes.c_int32), ("latent_dim", ctypes.c_int32)]


class IoWeights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("w_text", "w_img_in", "w_ref_in", "w_final", "w_out")]


class RopeLayout(ctypes.Structure):
    _fields_ = [("n_text", ctypes.c_int32), ("grid_h", ctypes.c_int32),
                ("grid_w", ctypes.c_int32), ("n_refs", ctypes.c_int32),
                ("ref_h", ctypes.POINTER(ctypes.c_int32)),
                ("ref_w", ctypes.POINTER(ctypes.c_int32)),
                ("theta", ctypes.c_double), ("hw_scale", ctypes.c_double)]


class KernelStats(ctypes.Structure):
    _fields_ = [("launches", ctypes.c_int64), ("total_ms", ctypes.c_double),
                ("tokens", ctypes.c_double), ("tokens_sq", ctypes.c_double)]


class DeviceInfo(ctypes.Structure):
    _fields_ = [("compute_units", ctypes.c_int32), ("clock_khz", ctypes.c_int32),
                ("bf16_dense_tflops", ctypes.c_double), ("arch", ctypes.c_char * 64)]


class WorkspaceLayout(ctypes.Structure):
    _fields_ = [("h", ctypes.c_size_t), ("q", ctypes.c_size_t), ("k", ctypes.c_size_t),
                ("vt", ctypes.c_size_t), ("cat", ctypes.c_size_t), ("part", ctypes.c_size_t),
                ("total", ctypes.c_size_t), ("n_pad", ctypes.c_int64)]


_lib = None


def load(path=LIB_PATH):
    """Load libflux3.so once and declare its signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"libflux3.so not built at {path}; build it with "
                          "python -m latent_flow_matching_flux_amd.build")
    lib = ctypes.CDLL(path)
    P = ctypes.POINTER
    i32, i64, sz, vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_void_p
    lib.flux3_layout_tokens.argtypes = [P(RopeLayout)]
    lib.flux3_layout_tokens.restype = i64
    lib.flux3_rope_tables_build.argtypes = [P(RopeLayout), vp, i64, vp]
    lib.flux3_rope_tables_build.restype = i32
    lib.flux3_workspace_bytes.argtypes = [P(Dims), i64]
    lib.flux3_workspace_bytes.restype = sz
    lib.flux3_workspace_layout_get.argtypes = [P(Dims), i64, P(WorkspaceLayout)]
    lib.flux3_workspace_layout_get.restype = i32
    lib.flux3_block_forward.argtypes = [P(Dims), P(BlockWeights), vp, i64, P(Segment), i32,
                                        vp, vp, vp, sz, vp]
    lib.flux3_block_forward.restype = i32
    lib.flux3_block_forward_noalloc.argtypes = [P(Dims), P(BlockWeights), vp, i64, P(Segment),
                                                i32, vp, vp, vp]
    lib.flux3_block_forward_noalloc.restype = i32
    lib.flux3_stack_forward.argtypes = [P(Dims), P(BlockWeights), i32, P(BlockWeights), i32,
                                        vp, i64, P(Segment), i32, vp, vp, i64, vp, vp, sz, vp]
    lib.flux3_stack_forward.restype = i32
    lib.flux3_weights_packed_bytes.argtypes = [P(Dims)]
    lib.flux3_weights_packed_bytes.restype = sz
    lib.flux3_weights_pack.argtypes = [P(Dims), P(BlockWeights), vp, sz, P(BlockWeights), vp]
    lib.flux3_weights_pack.restype = i32
    lib.flux3_weights_fp8r_bytes.argtypes = [P(Dims)]
    lib.flux3_weights_fp8r_bytes.restype = sz
    lib.flux3_weights_quantize_fp8r.argtypes = [P(Dims), P(BlockWeights), vp, sz,
                                                P(BlockWeights), vp]
    lib.flux3_weights_quantize_fp8r.restype = i32
    lib.flux3_transformer_workspace_bytes.argtypes = [P(Dims), P(IoDims), i64]
    lib.flux3_transformer_workspace_bytes.restype = sz
    lib.flux3_transformer_forward.argtypes = [P(Dims), P(IoDims), P(IoWeights),
                                              P(ModulationWeights), P(BlockWeights), i32,
                                              P(BlockWeights), i32, vp, vp, vp, P(Segment), i32,
                                              ctypes.c_float, ctypes.c_float, vp, vp, vp, sz, vp]
    lib.flux3_transformer_forward.restype = i32
    lib.flux3_sigmas.argtypes = [i32, ctypes.c_double, P(ctypes.c_float)]
    lib.flux3_sigmas.restype = i32
    lib.flux3_euler_step.argtypes = [vp, vp, vp, i64, ctypes.c_float, ctypes.c_float, vp]
    lib.flux3_euler_step.restype = i32
    lib.flux3_sample_workspace_bytes.argtypes = [P(Dims), P(IoDims), i64]
    lib.flux3_sample_workspace_bytes.restype = sz
    lib.flux3_sample.argtypes = [P(Dims), P(IoDims), P(IoWeights), P(ModulationWeights),
                                 P(BlockWeights), i32, P(BlockWeights), i32, vp, vp, vp,
                                 P(Segment), i32, i32, ctypes.c_double, i32, vp, vp, vp, sz, vp]
    lib.flux3_sample.restype = i32
    lib.flux3_modulation_workspace_bytes.argtypes = [P(Dims)]
    lib.flux3_modulation_workspace_bytes.restype = sz
    lib.flux3_modulation_forward.argtypes = [P(Dims), P(ModulationWeights), P(ctypes.c_float),
                                             ctypes.c_float, P(Segment), i32, vp, vp, sz, vp]
    lib.flux3_modulation_forward.restype = i32
    lib.flux3_profile_enable.argtypes = [i32]
    lib.flux3_profile_enable.restype = None
    lib.flux3_profile_reset.argtypes = []
    lib.flux3_profile_reset.restype = None
    lib.flux3_profile_read.argtypes = [i32, P(KernelStats)]
    lib.flux3_profile_read.restype = i32
    lib.flux3_profile_read_tokens.argtypes = [i32, i64, P(KernelStats)]
    lib.flux3_profile_read_tokens.restype = i32
    lib.flux3_device_query.argtypes = [i32, P(DeviceInfo)]
    lib.flux3_device_query.restype = i32
    lib.flux3_set_debug_sync.argtypes = [i32]
    lib.flux3_set_debug_sync.restype = None
    lib.flux3_status_string.argtypes = [i32]
    lib.flux3_status_string.restype = ctypes.c_char_p
    lib.flux3_last_error_detail.argtypes = []
    lib.flux3_last_error_detail.restype = ctypes.c_char_p
    _lib = lib
    return lib


def _check(status):
    if status != FLUX3_OK:
        detail = load().flux3_last_error_detail().decode()
        raise Flux3Error(status, detail)


def _ptr(t):
    """Device (or host) address of a tensor, an int address, or None -> NULL."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream_handle(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def make_dims(d):
    """Dims from any object with width/heads/head_dim/mlp_hidden."""
    if isinstance(d, Dims):
        return d
    return Dims(d.width, d.heads, d.head_dim, d.mlp_hidden)


def make_segments(segs):
    arr = (Segment * max(len(segs), 1))()
    for i, s in enumerate(segs):
        if hasattr(s, "start"):
            arr[i] = Segment(s.start, s.count, s.mode)
        else:
            arr[i] = Segment(*s)
    return arr, len(segs)


def make_weights(w):
    """BlockWeights from a dict of tensors (keys as in the header struct; an
    optional "layout" entry, default WEIGHTS_LINEAR; "s_proj" and "s_out"
    for WEIGHTS_FP8R)."""
    if isinstance(w, BlockWeights):
        return w
    return BlockWeights(*[_ptr(w.get(k)) for k in MATRICES + ("q_norm", "k_norm")],
                        int(w.get("layout", WEIGHTS_LINEAR)), _ptr(w.get("s_proj")),
                        _ptr(w.get("s_out")))


def weights_packed_bytes(dims):
    return load().flux3_weights_packed_bytes(ctypes.byref(make_dims(dims)))


def weights_pack(dims, w, buffer, stream=None):
    """flux3_weights_pack: copy a block's Linear-layout matrices into buffer
    (device, >= weights_packed_bytes(dims) bytes) in the packed operand
    layout.  Returns the BlockWeights pointing into buffer (layout
    WEIGHTS_PACKED); buffer must stay alive while it is used."""
    out = BlockWeights()
    _check(load().flux3_weights_pack(ctypes.byref(make_dims(dims)), ctypes.byref(make_weights(w)),
                                     _ptr(buffer), buffer.numel() * buffer.element_size()
                                     if hasattr(buffer, "numel") else 0,
                                     ctypes.byref(out), _stream_handle(stream)))
    # the struct points into buffer and at the caller's norm vectors
    out._keep = (buffer, w.get("q_norm"), w.get("k_norm")) if isinstance(w, dict) else (buffer, w)
    return out


def weights_fp8r_bytes(dims):
    return load().flux3_weights_fp8r_bytes(ctypes.byref(make_dims(dims)))


def weights_quantize_fp8r(dims, w, buffer, stream=None):
    """flux3_weights_quantize_fp8r: the rowwise-FP8 form of a block's
    Linear-layout weights, written into buffer (device, >=
    weights_fp8r_bytes(dims) bytes).  Returns the BlockWeights pointing into
    buffer (layout WEIGHTS_FP8R); buffer must stay alive while it is used."""
    out = BlockWeights()
    _check(load().flux3_weights_quantize_fp8r(
        ctypes.byref(make_dims(dims)), ctypes.byref(make_weights(w)), _ptr(buffer),
        buffer.numel() * buffer.element_size() if hasattr(buffer, "numel") else 0,
        ctypes.byref(out), _stream_handle(stream)))
    out._keep = (buffer, w.get("q_norm"), w.get("k_norm")) if isinstance(w, dict) else (buffer, w)
    return out


def make_layout(lay):
    """RopeLayout from an object with n_text, grid_h, grid_w, refs, theta,
    hw_scale.  Keeps the ref arrays alive on the returned struct."""
    refs = list(getattr(lay, "refs", ()))
    rh = (ctypes.c_int32 * max(len(refs), 1))(*[r[0] for r in refs])
    rw = (ctypes.c_int32 * max(len(refs), 1))(*[r[1] for r in refs])
    out = RopeLayout(lay.n_text, lay.grid_h, lay.grid_w, len(refs),
                     ctypes.cast(rh, ctypes.POINTER(ctypes.c_int32)),
                     ctypes.cast(rw, ctypes.POINTER(ctypes.c_int32)),
                     float(lay.theta), float(lay.hw_scale))
    out._keep = (rh, rw)
    return out


def layout_tokens(lay):
    return load().flux3_layout_tokens(ctypes.byref(make_layout(lay)))


def rope_tables_build(lay, rope, n_tokens=None, stream=None):
    """flux3_rope_tables_build: fill rope [N][64][2] fp32 for a layout."""
    L = make_layout(lay)
    if n_tokens is None:
        n_tokens = rope.shape[0] if rope is not None else 0
    _check(load().flux3_rope_tables_build(ctypes.byref(L), _ptr(rope), n_tokens,
                                          _stream_handle(stream)))


def workspace_bytes(dims, n_tokens):
    return load().flux3_workspace_bytes(ctypes.byref(make_dims(dims)), n_tokens)


def workspace_layout(dims, n_tokens):
    out = WorkspaceLayout()
    _check(load().flux3_workspace_layout_get(ctypes.byref(make_dims(dims)), n_tokens,
                                             ctypes.byref(out)))
    return out


def block_forward(dims, w, x, segs, mod, rope, workspace, n_tokens=None,
                  workspace_nbytes=None, stream=None):
    """flux3_block_forward: one block in place on x [N][D] fp32."""
    seg_arr, n_segs = make_segments(segs)
    W = make_weights(w)
    if n_tokens is None:
        n_tokens = x.shape[0]
    if workspace_nbytes is None:
        workspace_nbytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(load().flux3_block_forward(ctypes.byref(make_dims(dims)), ctypes.byref(W), _ptr(x),
                                      n_tokens, seg_arr, n_segs, _ptr(mod), _ptr(rope),
                                      _ptr(workspace), workspace_nbytes, _stream_handle(stream)))


def block_forward_noalloc(dims, w, x, segs, mod, rope, n_tokens=None, stream=None):
    """flux3_block_forward_noalloc: one block in place on x [N][D] fp32 with
    the library's own fixed intermediates (no workspace; N limited to what
    NOALLOC_SCRATCH_BYTES holds)."""
    seg_arr, n_segs = make_segments(segs)
    W = make_weights(w)
    if n_tokens is None:
        n_tokens = x.shape[0]
    _check(load().flux3_block_forward_noalloc(ctypes.byref(make_dims(dims)), ctypes.byref(W),
                                              _ptr(x), n_tokens, seg_arr, n_segs, _ptr(mod),
                                              _ptr(rope), _stream_handle(stream)))


def stack_forward(dims, per_mode, joint, x, segs, mod_stage1, mod_stage2, rope, workspace,
                  mod_block_stride=0, n_tokens=None, workspace_nbytes=None, stream=None):
    """flux3_stack_forward.  per_mode: {mode: [weights dict, ...]} (equal
    lengths) or a flat list of 3*n_pm weights; joint: list of weights."""
    pm_arr, n_pm, j_arr, n_joint = _block_arrays(per_mode, joint)
    seg_arr, n_segs = make_segments(segs)
    if n_tokens is None:
        n_tokens = x.shape[0]
    if workspace_nbytes is None:
        workspace_nbytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(load().flux3_stack_forward(ctypes.byref(make_dims(dims)), pm_arr, n_pm, j_arr,
                                      n_joint, _ptr(x), n_tokens, seg_arr, n_segs,
                                      _ptr(mod_stage1), _ptr(mod_stage2), mod_block_stride,
                                      _ptr(rope), _ptr(workspace), workspace_nbytes,
                                      _stream_handle(stream)))


def modulation_workspace_bytes(dims):
    return load().flux3_modulation_workspace_bytes(ctypes.byref(make_dims(dims)))


def modulation_forward(dims, w, t_by_mode, segs, mod, workspace, t_target=None,
                       workspace_nbytes=None, stream=None):
    """flux3_modulation_forward: one stage's [n_segs][3][width] modulation
    vectors from timesteps.  w: dict with w1, w2, optional w1_tgt, w2_tgt,
    and w_mod (a {mode: tensor} dict or a 3-list, None for unused modes);
    t_by_mode: 3 timesteps (text, image, reference)."""
    W = _modulation_weights(w)
    t = (ctypes.c_float * 3)(*[float(v) for v in t_by_mode])
    seg_arr, n_segs = make_segments(segs)
    if workspace_nbytes is None:
        workspace_nbytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(load().flux3_modulation_forward(ctypes.byref(make_dims(dims)), ctypes.byref(W), t,
                                           -1.0 if t_target is None else float(t_target),
                                           seg_arr, n_segs, _ptr(mod), _ptr(workspace),
                                           workspace_nbytes, _stream_handle(stream)))


def _modulation_weights(w):
    wm = w.get("w_mod", {})
    mods = [wm.get(m) if isinstance(wm, dict) else wm[m] for m in range(3)]
    return ModulationWeights(_ptr(w.get("w1")), _ptr(w.get("w2")), _ptr(w.get("w1_tgt")),
                             _ptr(w.get("w2_tgt")), (ctypes.c_void_p * 3)(*[_ptr(t) for t in mods]))


def make_io_dims(d):
    if isinstance(d, IoDims):
        return d
    return IoDims(d.text_dim, d.latent_dim)


def transformer_workspace_bytes(dims, io_dims, n_tokens):
    return load().flux3_transformer_workspace_bytes(ctypes.byref(make_dims(dims)),
                                                    ctypes.byref(make_io_dims(io_dims)), n_tokens)


def _block_arrays(per_mode, joint):
    if isinstance(per_mode, dict):
        n_pm = max((len(v) for v in per_mode.values()), default=0)
        flat = []
        for m in range(3):
            blocks = per_mode.get(m, [])
            for b in range(n_pm):
                flat.append(make_weights(blocks[b]) if b < len(blocks) else BlockWeights())
    else:
        flat = [make_weights(w) for w in per_mode]
        n_pm = len(flat) // 3
    pm_arr = (BlockWeights * max(len(flat), 1))(*flat)
    jt = [make_weights(w) for w in joint]
    jt_arr = (BlockWeights * max(len(jt), 1))(*jt)
    return pm_arr, n_pm, jt_arr, len(jt)


def transformer_forward(dims, io_dims, io_w, mod_w, per_mode, joint, text, image, refs, segs, t,
                        rope, velocity, workspace, t_target=None, workspace_nbytes=None,
                        stream=None):
    """flux3_transformer_forward.  io_w: dict with w_text, w_img_in, w_ref_in,
    w_final, w_out; mod_w: two modulation weight dicts (stage 1, stage 2) as
    for modulation_forward; per_mode / joint as for stack_forward."""
    io = IoWeights(*[_ptr(io_w.get(k)) for k in ("w_text", "w_img_in", "w_ref_in", "w_final",
                                                  "w_out")])
    mw = (ModulationWeights * 2)(_modulation_weights(mod_w[0]), _modulation_weights(mod_w[1]))
    pm_arr, n_pm, jt_arr, n_joint = _block_arrays(per_mode, joint)
    seg_arr, n_segs = make_segments(segs)
    if workspace_nbytes is None:
        workspace_nbytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(load().flux3_transformer_forward(
        ctypes.byref(make_dims(dims)), ctypes.byref(make_io_dims(io_dims)), ctypes.byref(io), mw,
        pm_arr, n_pm, jt_arr, n_joint, _ptr(text), _ptr(image), _ptr(refs), seg_arr, n_segs,
        float(t), -1.0 if t_target is None else float(t_target), _ptr(rope), _ptr(velocity),
        _ptr(workspace), workspace_nbytes, _stream_handle(stream)))


def sigmas(steps, shift=6.93):
    """flux3_sigmas: the shifted schedule, a list of steps + 1 floats."""
    out = (ctypes.c_float * (steps + 1))()
    _check(load().flux3_sigmas(int(steps), float(shift), out))
    return list(out)


def euler_step(v, latent, sigma, sigma_next, x0_preview=None, stream=None):
    """flux3_euler_step on fp32 device tensors (in place on latent)."""
    _check(load().flux3_euler_step(_ptr(v), _ptr(latent), _ptr(x0_preview), latent.numel(),
                                   float(sigma), float(sigma_next), _stream_handle(stream)))


def sample_workspace_bytes(dims, io_dims, n_tokens):
    return load().flux3_sample_workspace_bytes(ctypes.byref(make_dims(dims)),
                                               ctypes.byref(make_io_dims(io_dims)), n_tokens)


def sample(dims, io_dims, io_w, mod_w, per_mode, joint, text, latent, refs, segs, steps, rope,
           workspace, shift=6.93, distilled=True, previews=None, workspace_nbytes=None,
           stream=None):
    """flux3_sample: the whole denoise loop, in place on latent."""
    io = IoWeights(*[_ptr(io_w.get(k)) for k in ("w_text", "w_img_in", "w_ref_in", "w_final",
                                                  "w_out")])
    mw = (ModulationWeights * 2)(_modulation_weights(mod_w[0]), _modulation_weights(mod_w[1]))
    pm_arr, n_pm, jt_arr, n_joint = _block_arrays(per_mode, joint)
    seg_arr, n_segs = make_segments(segs)
    if workspace_nbytes is None:
        workspace_nbytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(load().flux3_sample(
        ctypes.byref(make_dims(dims)), ctypes.byref(make_io_dims(io_dims)), ctypes.byref(io), mw,
        pm_arr, n_pm, jt_arr, n_joint, _ptr(text), _ptr(latent), _ptr(refs), seg_arr, n_segs,
        int(steps), float(shift), 1 if distilled else 0, _ptr(rope), _ptr(previews),
        _ptr(workspace), workspace_nbytes, _stream_handle(stream)))


def profile_enable(on):
    load().flux3_profile_enable(1 if on else 0)


def profile_reset():
    load().flux3_profile_reset()


def profile_read(kernel, n_tokens=None):
    """Stats for one kernel kind (name from KERNELS or its index): dict with
    launches, total_ms, tokens (sum of M), tokens_sq (sum of M^2); with
    n_tokens, over the launches with M == n_tokens only."""
    idx = KERNELS.index(kernel) if isinstance(kernel, str) else int(kernel)
    out = KernelStats()
    if n_tokens is None:
        _check(load().flux3_profile_read(idx, ctypes.byref(out)))
    else:
        _check(load().flux3_profile_read_tokens(idx, n_tokens, ctypes.byref(out)))
    return {"launches": out.launches, "total_ms": out.total_ms, "tokens": out.tokens,
            "tokens_sq": out.tokens_sq}


def device_query(device=0):
    """flux3_device_query: CU count, clock, arch and the implied bf16 MFMA peak."""
    out = DeviceInfo()
    _check(load().flux3_device_query(device, ctypes.byref(out)))
    return {"compute_units": out.compute_units, "clock_khz": out.clock_khz,
            "bf16_dense_tflops": out.bf16_dense_tflops, "arch": out.arch.decode()}


def set_debug_sync(on):
    load().flux3_set_debug_sync(1 if on else 0)


def status_string(status):
    return load().flux3_status_string(status).decode()
