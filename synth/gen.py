"""Seeded random draws for block inputs.

Every tensor comes from its own NumPy PCG64 stream keyed by
(seed, block_id, tensor_id), so any one block's weights can be regenerated
without drawing the others.  Weights are drawn in fp32 from N(0, 0.02^2) and
rounded once to bfloat16 (round to nearest, ties to even); both the GPU path
and the oracle consume those same bf16 values.

The modulation vectors (shift, scale, gate per token segment) are drawn
directly as N(0, MOD_STD^2) stand-ins for the output of the timestep
embedding path; computing them from a timestep is a separate step that the
hot path takes as an input.
"""
import numpy as np

WEIGHT_STD = 0.02
MOD_STD = 0.07

# tensor ids inside one block
T_WQ, T_WK, T_WV, T_WO, T_WGATE, T_WUP, T_WDOWN, T_QNORM, T_KNORM = range(9)
# stream ids for non-weight tensors (block_id slot)
_X_STREAM = 1_000_000
_MOD_STREAM = 2_000_000
_TIME_STREAM = 3_000_000   # timestep embedder and modulation linears
# tensor ids of the timestep path
T_EMB_W1, T_EMB_W2, T_TGT_W1, T_TGT_W2 = range(4)
T_WMOD0 = 10               # + 3 * stage + mode


def _rng(*key):
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(list(key))))


def bf16_round_bits(a):
    """fp32 array -> uint16 bfloat16 bit patterns, round to nearest even."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(bits):
    """uint16 bfloat16 bit patterns -> fp32 (exact)."""
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << 16).view(np.float32)


def _normal_bf16(shape, std, *key):
    a = _rng(*key).standard_normal(int(np.prod(shape)), dtype=np.float32)
    a *= np.float32(std)
    return bf16_round_bits(a).reshape(shape)


def block_weights(seed, block_id, dims, norm_stress=False, std=WEIGHT_STD):
    """One block's weights, torch-Linear layout [out][in], as bf16 bits.

    Returns a dict with uint16 arrays wq, wk, wv, wo [D][D], w_gate, w_up
    [F][D], w_down [D][F], and float32 q_norm, k_norm [head_dim] (all ones
    unless norm_stress, which draws 1 + N(0, 0.1^2)).
    """
    D, F, hd = dims.width, dims.mlp_hidden, dims.head_dim
    w = {
        "wq": _normal_bf16((D, D), std, seed, block_id, T_WQ),
        "wk": _normal_bf16((D, D), std, seed, block_id, T_WK),
        "wv": _normal_bf16((D, D), std, seed, block_id, T_WV),
        "wo": _normal_bf16((D, D), std, seed, block_id, T_WO),
        "w_gate": _normal_bf16((F, D), std, seed, block_id, T_WGATE),
        "w_up": _normal_bf16((F, D), std, seed, block_id, T_WUP),
        "w_down": _normal_bf16((D, F), std, seed, block_id, T_WDOWN),
    }
    if norm_stress:
        w["q_norm"] = (1.0 + 0.1 * _rng(seed, block_id, T_QNORM).standard_normal(hd)).astype(np.float32)
        w["k_norm"] = (1.0 + 0.1 * _rng(seed, block_id, T_KNORM).standard_normal(hd)).astype(np.float32)
    else:
        w["q_norm"] = np.ones(hd, np.float32)
        w["k_norm"] = np.ones(hd, np.float32)
    return w


def modulation_weights(seed, width, stages=(0,), modes=(0, 1, 2), target=False,
                       std=WEIGHT_STD):
    """Weights of the timestep path as bf16 bits, torch-Linear layout: the
    embedder w1 [width][256], w2 [width][width]; with target, the flow-map
    target embedder w1_tgt, w2_tgt; and w_mod[stage][mode] [3*width][width]
    for the listed stages and modes.  All N(0, std^2) before rounding."""
    D = width
    w = {"w1": _normal_bf16((D, 256), std, seed, _TIME_STREAM, T_EMB_W1),
         "w2": _normal_bf16((D, D), std, seed, _TIME_STREAM, T_EMB_W2)}
    if target:
        w["w1_tgt"] = _normal_bf16((D, 256), std, seed, _TIME_STREAM, T_TGT_W1)
        w["w2_tgt"] = _normal_bf16((D, D), std, seed, _TIME_STREAM, T_TGT_W2)
    w["w_mod"] = {st: {m: _normal_bf16((3 * D, D), std, seed, _TIME_STREAM, T_WMOD0 + 3 * st + m)
                       for m in modes} for st in stages}
    return w


def tokens(seed, n, width):
    """Residual-stream input x ~ N(0, 1), fp32 [n][width]."""
    return _rng(seed, _X_STREAM, n, width).standard_normal((n, width), dtype=np.float32)


def modulation(seed, stream, n_segs, width, std=MOD_STD):
    """(shift, scale, gate) per segment: fp32 [n_segs][3][width] ~ N(0, std^2)."""
    a = _rng(seed, _MOD_STREAM, stream, n_segs, width).standard_normal(
        (n_segs, 3, width), dtype=np.float32)
    return a * np.float32(std)


# the linears around the stack and the call's edge inputs
_IO_STREAM = 4_000_000
T_IO_TEXT, T_IO_IMG, T_IO_REF, T_IO_FINAL, T_IO_OUT = range(5)
_EDGE_STREAM = 5_000_000
T_IN_TEXT, T_IN_IMAGE, T_IN_REFS = range(3)
TEXT_DIM, LATENT_DIM = 20480, 128


def io_weights(seed, width, text_dim=TEXT_DIM, latent_dim=LATENT_DIM, std=WEIGHT_STD):
    """The transformer call's own linears as bf16 bits, torch-Linear layout:
    w_text [width][text_dim], w_img_in and w_ref_in [width][latent_dim],
    w_final [2*width][width], w_out [latent_dim][width]; N(0, std^2)."""
    D = width
    return {"w_text": _normal_bf16((D, text_dim), std, seed, _IO_STREAM, T_IO_TEXT),
            "w_img_in": _normal_bf16((D, latent_dim), std, seed, _IO_STREAM, T_IO_IMG),
            "w_ref_in": _normal_bf16((D, latent_dim), std, seed, _IO_STREAM, T_IO_REF),
            "w_final": _normal_bf16((2 * D, D), std, seed, _IO_STREAM, T_IO_FINAL),
            "w_out": _normal_bf16((latent_dim, D), std, seed, _IO_STREAM, T_IO_OUT)}


def edge_inputs(seed, n_text, n_image, n_ref, text_dim=TEXT_DIM, latent_dim=LATENT_DIM):
    """Inputs of one transformer call: text-encoder vectors as bf16 bits
    [n_text][text_dim] ~ N(0, 1); noisy-image and reference latent tokens
    [n][latent_dim] ~ N(0, 1) in fp32, rounded to bf16-representable values
    (the call rounds them to bf16 on the device, exactly, then)."""
    text = _normal_bf16((n_text, text_dim), 1.0, seed, _EDGE_STREAM, T_IN_TEXT)
    img = bf16_bits_to_f32(_normal_bf16((n_image, latent_dim), 1.0, seed, _EDGE_STREAM, T_IN_IMAGE))
    refs = bf16_bits_to_f32(_normal_bf16((n_ref, latent_dim), 1.0, seed, _EDGE_STREAM, T_IN_REFS))
    return text, img, refs
