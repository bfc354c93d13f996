"""Plain CPU oracle for the FLUX.3 Image Klein transformer block.

TEST INFRASTRUCTURE ONLY.  This module is the correctness reference that the
HIP path is compared against.  Only the test suite, the package entry's
smoke check and the benchmark's CPU-baseline leg may import or call it; the
product path never does, and nothing here is shared with the HIP kernels or
their host code.

Sources (the release pages; cited by page title and section):

* [P1]  "FLUX.3 Image Klein Is Now Available in Diffusers" (15jq.com),
        sections "Speed, architecture, and how the tokens move" and
        "Smaller GPUs, single files, and custom LoRA training" (rowwise FP8).
* [P3]  The Chinese translation of the Diffusers release post (everytik.com):
        the block listing (modulated by shift, scale and gate) and the RoPE position
        table under the model walk-through.
* [P4]  "How to Run FLUX 3 Image Klein Locally" (rohitghumare.com), sections
        "Inside the transformer", "The latent space and the VAE",
        "What step distillation removed", "What Black Forest Labs released".
* [P5]  The ifeeling.app summary, architecture paragraphs (reference offset
        runs negatively along l).

Readings where the pages are silent (each is a parameter or a documented
constant): LayerNorm/RMSNorm epsilon 1e-6; RMSNorm per 128-dim head with a
learned [128] scale; RoPE base theta = 10000 with adjacent pairs (2i, 2i+1)
and axis a owning head dims [32a, 32a+32); image/reference h, w = row/2,
col/2 taken as real division on the token-grid index (hw_scale = 0.5);
attention scale 1/sqrt(128); an output projection after attention; no
biases; SwiGLU with silu on the gate branch; shift, scale, gate order.
Around the stack: separate input linears for image and reference latent
tokens; an output layer of LayerNorm (no affine), (shift, scale) from a
D -> 2D linear of the image timestep's embedding, and a D -> 128 linear.

Precision: float64 by default (pass dtype=np.float32 for the large timing
runs).  Every function follows its definition directly; the only blocking is
an optional split of attention over independent query rows, which does not
change any sum.

Parity status per function (pins live in tests/test_oracle_pins.py):
  token_positions, rope_tables, apply_rope, layer_norm, modulate,
  rms_norm_heads, attention, silu, swiglu_mlp, block_forward,
  block_forward_rows, stack_forward, timestep_embedding,
  modulation_from_t, shifted_sigmas, euler_step, x0_preview, sample,
  input_projection, final_modulation, output_layer, transformer_forward,
  e4m3_values, e4m3_encode, quantize_rowwise, dequantize_rowwise,
  fake_quantize_rows, fused_block_matrices, quantize_block_weights,
  block_forward_quantized, block_forward_fp8: all pinned.
"""
import numpy as np

EPS_LN = 1e-6
EPS_RMS = 1e-6
THETA = 10000.0
HW_SCALE = 0.5
ROPE_AXES = 4          # (t, h, w, l)   [P1], [P3] RoPE table
AXIS_DIM = 32          # a quarter of each 128-dim head per axis   [P1]

MODE_TEXT, MODE_IMAGE, MODE_REF = 0, 1, 2


# --------------------------------------------------------------------------
# helpers
# --------------------------------------------------------------------------
def as_float(a, dtype=np.float64):
    """Weights arrive either as float arrays or as bfloat16 bit patterns
    (uint16).  A bfloat16 value is the upper half of an IEEE binary32, so
    the bits are widened by a 16-bit shift and reinterpreted."""
    a = np.asarray(a)
    if a.dtype == np.uint16:
        a = (a.astype(np.uint32) << 16).view(np.float32)
    return a.astype(dtype)


# --------------------------------------------------------------------------
# positions and rotary tables    [P1] RoPE paragraph, [P3] RoPE table, [P5]
# --------------------------------------------------------------------------
def token_positions(n_text, grid_h, grid_w, refs=(), hw_scale=HW_SCALE):
    """(t, h, w, l) for every token, in sequence order [text | image | refs].

    Text token i sits at (0, 0, 0, i).  The noisy-image token at grid
    (row, col) sits at (0, row/2, col/2, 0).  Token (row, col) of reference
    k (0-based) sits at (0, row/2, col/2, -(k+1)).  Image rows are in raster
    order (row-major), the flattening of the packed latent grid [P4 "The
    latent space and the VAE"].  hw_scale=0.5 is the row/2 reading.
    """
    pos = []
    for i in range(n_text):
        pos.append((0.0, 0.0, 0.0, float(i)))
    for row in range(grid_h):
        for col in range(grid_w):
            pos.append((0.0, row * hw_scale, col * hw_scale, 0.0))
    for k, (rh, rw) in enumerate(refs):
        for row in range(rh):
            for col in range(rw):
                pos.append((0.0, row * hw_scale, col * hw_scale, float(-(k + 1))))
    return np.array(pos, dtype=np.float64).reshape(-1, 4)


def rope_tables(positions, theta=THETA):
    """cos/sin table [N][64][2] in float32, computed in float64, rounded once.

    Pair p = 16*a + j of a head belongs to axis a (t, h, w, l) and rotates
    by angle positions[:, a] * theta**(-2j/32): the standard rotary
    frequencies over a 32-dim sub-space, one sub-space per axis [P1].
    """
    positions = np.asarray(positions, dtype=np.float64)
    n = positions.shape[0]
    half = AXIS_DIM // 2
    table = np.zeros((n, ROPE_AXES * half, 2), dtype=np.float64)
    for a in range(ROPE_AXES):
        for j in range(half):
            omega = theta ** (-2.0 * j / AXIS_DIM)
            phi = positions[:, a] * omega
            table[:, a * half + j, 0] = np.cos(phi)
            table[:, a * half + j, 1] = np.sin(phi)
    return table.astype(np.float32)


def apply_rope(x, table):
    """Rotate each adjacent pair (2p, 2p+1) of every head by the table angle.

    x: [N][H][128]; table: [N][64][2] (cos, sin).  (x0, x1) becomes
    (x0 cos - x1 sin, x0 sin + x1 cos).
    """
    x = np.asarray(x)
    cos = np.asarray(table[:, None, :, 0], dtype=x.dtype)
    sin = np.asarray(table[:, None, :, 1], dtype=x.dtype)
    x0 = x[..., 0::2]
    x1 = x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = x0 * cos - x1 * sin
    out[..., 1::2] = x0 * sin + x1 * cos
    return out


# --------------------------------------------------------------------------
# block pieces    [P3] block listing, [P1], [P4 "Inside the transformer"]
# --------------------------------------------------------------------------
def layer_norm(x, eps=EPS_LN):
    """LayerNorm over the last axis with no learned scale or shift."""
    mu = x.mean(axis=-1, keepdims=True)
    var = ((x - mu) ** 2).mean(axis=-1, keepdims=True)
    return (x - mu) / np.sqrt(var + eps)


def modulate(hhat, shift, scale):
    """adaLN modulation (1 + scale) * h + shift."""
    return (1.0 + scale) * hhat + shift


def rms_norm_heads(x, weight, eps=EPS_RMS):
    """RMS normalisation over each head's 128 dims, times a [128] scale."""
    ms = (x ** 2).mean(axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * weight


# Attention's heads and query chunks are independent computations; they may
# be evaluated by THREADS threads at once (numpy releases the GIL inside its
# kernels, and the BLAS library is held to one thread per call meanwhile).
# Every piece runs the same operations either way; THREADS only changes how
# long the oracle takes (and, at most, the BLAS library's own blocking).
THREADS = 1


def attention(q, k, v, chunk=None):
    """Full bidirectional softmax attention per head, no mask.

    q, k, v: [N][H][128] (q may have fewer rows than k, v).  Scores are
    q.k / sqrt(128), softmax over all keys (max subtracted), times v.
    Returns [Nq][H][128].  chunk splits the query rows (each row's softmax
    is still taken over every key in one piece).
    """
    nq, n_heads, hd = q.shape
    scale = 1.0 / np.sqrt(hd)
    out = np.empty((nq, n_heads, hd), dtype=q.dtype)
    step = max(nq if not chunk else chunk, 1)

    def piece(h, r0):
        kh = k[:, h, :]
        vh = v[:, h, :]
        qh = q[r0:r0 + step, h, :]
        s = (qh @ kh.T) * scale
        s = s - s.max(axis=-1, keepdims=True)
        p = np.exp(s)
        p = p / p.sum(axis=-1, keepdims=True)
        out[r0:r0 + step, h, :] = p @ vh

    jobs = [(h, r0) for h in range(n_heads) for r0 in range(0, nq, step)]
    if THREADS > 1 and len(jobs) > 1:
        from concurrent.futures import ThreadPoolExecutor
        from threadpoolctl import threadpool_limits
        with threadpool_limits(limits=1, user_api="blas"), ThreadPoolExecutor(THREADS) as ex:
            for f in [ex.submit(piece, h, r0) for h, r0 in jobs]:
                f.result()
    else:
        for h, r0 in jobs:
            piece(h, r0)
    return out


def silu(z):
    """z * sigmoid(z)."""
    return z / (1.0 + np.exp(-z))


def swiglu_mlp(h, w_gate, w_up, w_down):
    """SwiGLU feed-forward: (silu(h W_gate^T) * (h W_up^T)) W_down^T."""
    return (silu(h @ w_gate.T) * (h @ w_up.T)) @ w_down.T


def _row_modulation(segs, mod, n, dtype):
    """Expand per-segment (shift, scale, gate) to per-row arrays [N][D]."""
    mod = np.asarray(mod, dtype=dtype)
    width = mod.shape[-1]
    shift = np.zeros((n, width), dtype)
    scale = np.zeros((n, width), dtype)
    gate = np.zeros((n, width), dtype)
    covered = np.zeros(n, bool)
    for s, (start, count, _mode) in enumerate(segs):
        shift[start:start + count] = mod[s, 0]
        scale[start:start + count] = mod[s, 1]
        gate[start:start + count] = mod[s, 2]
        covered[start:start + count] = True
    if not covered.all():
        raise ValueError("segments must cover every token")
    return shift, scale, gate


def _weights(w, dtype):
    return {name: as_float(val, dtype) for name, val in w.items()}


def block_forward(x, w, segs, mod, rope, heads=None, dtype=np.float64,
                  eps_ln=EPS_LN, eps_rms=EPS_RMS, keep=False, attn_chunk=None):
    """One transformer block, in the order of the model walk-through of the
    Diffusers release post ([P3], its block section; [P4] "Inside the
    transformer"):

      h   = (1 + c_scale) . LN(x) + c_shift     LN without affine; c per segment
      Q   = R(N_q(h Wq^T)),  K = R(N_k(h Wk^T)),  V = h Wv^T
            (N: per-head RMS normalisation with a [128] scale, R: 4-axis rotation)
      A   = softmax(Q K^T / sqrt(128)) V  per head, then A Wo^T
      G   = (silu(h Wg^T) * (h Wu^T)) Wd^T     (SwiGLU, beside attention)
      x'  = x + c_gate . (A Wo^T + G)

    x: [N][D]; w: dict of weights (torch Linear layout [out][in]); segs:
    list of (start, count, mode) covering [0, N); mod: [n_segs][3][D]
    (shift, scale, gate) for each segment -- each token type gets its own
    vectors [P1]; rope: [N][64][2] table.  keep=True also returns the
    intermediates {h, q, k, v, o, act, out}.
    """
    x = np.asarray(x, dtype=dtype)
    n, width = x.shape
    wf = _weights(w, dtype)
    hd = wf["q_norm"].shape[0]
    if heads is None:
        heads = width // hd
    shift, scale, gate = _row_modulation(segs, mod, n, dtype)

    h = modulate(layer_norm(x, eps_ln), shift, scale)
    q = (h @ wf["wq"].T).reshape(n, heads, hd)
    k = (h @ wf["wk"].T).reshape(n, heads, hd)
    v = (h @ wf["wv"].T).reshape(n, heads, hd)
    q = apply_rope(rms_norm_heads(q, wf["q_norm"], eps_rms), rope)
    k = apply_rope(rms_norm_heads(k, wf["k_norm"], eps_rms), rope)
    o = attention(q, k, v, chunk=attn_chunk).reshape(n, width)
    a = o @ wf["wo"].T
    act = silu(h @ wf["w_gate"].T) * (h @ wf["w_up"].T)
    m = act @ wf["w_down"].T
    out = a + m
    x_new = x + gate * out
    if keep:
        return x_new, {"h": h, "q": q, "k": k, "v": v, "o": o, "act": act,
                       "out": out}
    return x_new


def block_forward_rows(x, w, segs, mod, rope, rows, heads=None,
                       dtype=np.float64, eps_ln=EPS_LN, eps_rms=EPS_RMS,
                       attn_chunk=None):
    """block_forward evaluated only at the output rows listed in `rows`.

    The same steps as block_forward: keys and values are computed for every
    token (attention reads all of them), queries, attention, the MLP and
    the residual only for the requested rows.  Returns [len(rows)][D].
    """
    x = np.asarray(x, dtype=dtype)
    rows = np.asarray(rows, dtype=np.int64)
    n, width = x.shape
    wf = _weights(w, dtype)
    hd = wf["q_norm"].shape[0]
    if heads is None:
        heads = width // hd
    shift, scale, gate = _row_modulation(segs, mod, n, dtype)

    h = modulate(layer_norm(x, eps_ln), shift, scale)
    k = (h @ wf["wk"].T).reshape(n, heads, hd)
    v = (h @ wf["wv"].T).reshape(n, heads, hd)
    k = apply_rope(rms_norm_heads(k, wf["k_norm"], eps_rms), rope)
    hr = h[rows]
    q = (hr @ wf["wq"].T).reshape(len(rows), heads, hd)
    q = apply_rope(rms_norm_heads(q, wf["q_norm"], eps_rms), rope[rows])
    o = attention(q, k, v, chunk=attn_chunk).reshape(len(rows), width)
    out = o @ wf["wo"].T + swiglu_mlp(hr, wf["w_gate"], wf["w_up"], wf["w_down"])
    return x[rows] + gate[rows] * out


def stack_forward(x, per_mode, joint, segs, mod_stage1, mod_stage2, rope,
                  dtype=np.float64, per_block_mod=False, block_fn=None):
    """The two-stage stack [P1], [P4 "Inside the transformer"].

    Stage 1: every segment (stream) runs the per-mode blocks of its own mode
    on its rows alone, attending only to itself.  Stage 2: the concatenated
    sequence [text | image | refs] runs the joint blocks, all tokens sharing
    the weights while each segment keeps its own modulation.

    per_mode[mode] is a list of block weight dicts (5 each); joint is a list
    (28).  mod_stage1 / mod_stage2: [n_segs][3][D] shared by every block of
    the stage, or, with per_block_mod, [n_blocks][n_segs][3][D].
    block_fn: the block (block_forward by default; block_forward_fp8 for
    weights in the form quantize_block_weights gives).
    """
    block_fn = block_fn or block_forward
    out = np.array(x, dtype=dtype, copy=True)
    for s, (start, count, mode) in enumerate(segs):
        rows = slice(start, start + count)
        for b, wb in enumerate(per_mode[mode]):
            m1 = mod_stage1[b] if per_block_mod else mod_stage1
            out[rows] = block_fn(out[rows], wb, [(0, count, mode)],
                                 np.asarray(m1)[s:s + 1], rope[rows], dtype=dtype)
    for b, wb in enumerate(joint):
        m2 = mod_stage2[b] if per_block_mod else mod_stage2
        out = block_fn(out, wb, segs, m2, rope, dtype=dtype)
    return out


# --------------------------------------------------------------------------
# timestep modulation (input side of the hot path)
#   [P1] modulation paragraphs, [P4 "Inside the transformer",
#   "What step distillation removed"], [P3] sampler notes on sigma*1000
# --------------------------------------------------------------------------
def timestep_embedding(t, dim=256, max_period=10000.0):
    """Sinusoidal embedding of tau = 1000 * t: [cos(tau f_i), sin(tau f_i)],
    f_i = max_period**(-i/(dim/2)), i < dim/2 (the transformer positional
    encoding of Vaswani et al. applied to the timestep)."""
    half = dim // 2
    tau = 1000.0 * float(t)
    f = max_period ** (-np.arange(half, dtype=np.float64) / half)
    return np.concatenate([np.cos(tau * f), np.sin(tau * f)])


def modulation_from_t(t_by_mode, w1, w2, w_mod, t_target=None, w1_tgt=None,
                      w2_tgt=None, dtype=np.float64):
    """Per-mode (shift, scale, gate) from timesteps.

    The embedder is two bias-free layers 256 -> D -> D with silu between
    [P4 "What step distillation removed"].  Noisy-image tokens use the
    current t; text and reference tokens always use t = 0 [P1], so their
    vectors never depend on the image timestep.  The distilled flow map adds
    a second embedder's output for the target timestep to every mode
    [P4 same section].  w_mod[mode] maps silu(embedding) to 3*D, split in
    the order shift, scale, gate.  Returns {mode: [3][D]}.
    """
    w1, w2 = as_float(w1, dtype), as_float(w2, dtype)
    extra = 0.0
    if t_target is not None:
        extra = as_float(w2_tgt, dtype) @ silu(as_float(w1_tgt, dtype) @ timestep_embedding(t_target))
    out = {}
    for mode, t in t_by_mode.items():
        e = w2 @ silu(w1 @ timestep_embedding(t)) + extra
        m = as_float(w_mod[mode], dtype) @ silu(e)
        out[mode] = m.reshape(3, -1)
    return out


# --------------------------------------------------------------------------
# the whole transformer call around the stack
#   [P1] "Speed, architecture, and how the tokens move" (token kinds, the
#   20,480-value text vectors, image tokens of 128 values, dropping text and
#   references at the end); [P4] "The text encoder", "The latent space and
#   the VAE", "Inside the transformer", "What step distillation removed"
# --------------------------------------------------------------------------
def input_projection(text, image, refs, w_text, w_img_in, w_ref_in, dtype=np.float64):
    """Residual-stream input [text | image | refs] in the sequence order of
    stage 2: text vectors (8 stacked 2,560-value encoder states = 20,480)
    through the text linear, image and reference latent tokens (128 values)
    through their own input linears; no biases.  Returns [N][D]."""
    parts = []
    for a, w in ((text, w_text), (image, w_img_in), (refs, w_ref_in)):
        a = as_float(a, dtype)
        if a.shape[0]:
            parts.append(a @ as_float(w, dtype).T)
    return np.concatenate(parts, axis=0)


def final_modulation(t, w1, w2, w_final, t_target=None, w1_tgt=None, w2_tgt=None,
                     dtype=np.float64):
    """(shift, scale) of the output layer: the image timestep's embedding (plus
    the flow-map target embedding, which reaches the output layer too [P4
    "What step distillation removed"]) through silu and a bias-free D -> 2D
    linear, split shift then scale.  Returns [2][D]."""
    e = as_float(w2, dtype) @ silu(as_float(w1, dtype) @ timestep_embedding(t))
    if t_target is not None:
        e = e + as_float(w2_tgt, dtype) @ silu(as_float(w1_tgt, dtype) @ timestep_embedding(t_target))
    return (as_float(w_final, dtype) @ silu(e)).reshape(2, -1)


def output_layer(x_img, shift, scale, w_out, dtype=np.float64, eps=EPS_LN):
    """Image tokens only: LayerNorm without affine, the output modulation,
    then the bias-free D -> 128 linear back to latent-token size
    [P4 "Inside the transformer"].  Returns the velocity [n_img][128]."""
    h = modulate(layer_norm(as_float(x_img, dtype), eps), as_float(shift, dtype),
                 as_float(scale, dtype))
    return h @ as_float(w_out, dtype).T


def transformer_forward(text, image, refs, segs, io_w, emb_w, w_mod, per_mode, joint, rope,
                        t, t_target=None, dtype=np.float64, keep=False, block_fn=None):
    """One transformer call: input projections, the two stages' modulation
    from the timesteps (image tokens t, text and references 0), the two-stage
    stack, then the output layer on the image rows.

    io_w: {w_text, w_img_in, w_ref_in, w_final, w_out}; emb_w: {w1, w2} and,
    for the distilled model, {w1_tgt, w2_tgt}; w_mod[stage][mode] the
    per-(stage, mode) modulation linears.  segs: (start, count, mode) in the
    order text, image, references.  Returns the velocity of the image tokens
    (and, with keep, the residual stream after the stack).  block_fn: as for
    stack_forward.
    """
    x = input_projection(text, image, refs, io_w["w_text"], io_w["w_img_in"],
                         io_w["w_ref_in"], dtype)
    modes = sorted({m for _s, _c, m in segs})
    t_by_mode = {m: (t if m == MODE_IMAGE else 0.0) for m in modes}
    tgt = dict(t_target=t_target, w1_tgt=emb_w.get("w1_tgt"), w2_tgt=emb_w.get("w2_tgt"))
    mods = []
    for stage in range(2):
        per = modulation_from_t(t_by_mode, emb_w["w1"], emb_w["w2"], w_mod[stage],
                                dtype=dtype, **tgt)
        mods.append(np.stack([per[m] for _s, _c, m in segs]))
    x = stack_forward(x, per_mode, joint, segs, mods[0], mods[1], rope, dtype=dtype,
                      block_fn=block_fn)
    shift, scale = final_modulation(t, emb_w["w1"], emb_w["w2"], io_w["w_final"], dtype=dtype,
                                    **tgt)
    img = [(st, c) for st, c, m in segs if m == MODE_IMAGE]
    rows = np.concatenate([np.arange(st, st + c) for st, c in img])
    v = output_layer(x[rows], shift, scale, io_w["w_out"], dtype)
    return (v, x) if keep else v


# --------------------------------------------------------------------------
# sampler schedule (outside the block; pinned by printed values)
#   [P4 "The denoise loop", "What step distillation removed"]
# --------------------------------------------------------------------------
def shifted_sigmas(steps, shift=6.93):
    """steps noise levels evenly spaced from 1 down to 1/steps, each mapped
    through sigma' = shift*sigma / (1 + (shift - 1)*sigma), then a final 0."""
    sig = np.linspace(1.0, 1.0 / steps, steps)
    sig = shift * sig / (1.0 + (shift - 1.0) * sig)
    return np.concatenate([sig, [0.0]])


def euler_step(sample, v, sigma, sigma_next):
    """Flow-matching Euler update: sample + (sigma_next - sigma) * v."""
    return sample + (sigma_next - sigma) * v


def x0_preview(sample, v, sigma):
    """The model's current guess of the clean latent: sample - sigma * v
    [P4 "The denoise loop"; the preview step of the Diffusers post]."""
    return sample - sigma * v


def sample(noise, text, refs, segs, io_w, emb_w, w_mod, per_mode, joint, rope, steps=16,
           shift=6.93, distilled=True, dtype=np.float64):
    """The denoise loop [P4 "The denoise loop", "What step distillation
    removed"]: start from pure noise at sigma = 1, and at each step call the
    transformer at the current sigma (the distilled flow map is also told the
    sigma it jumps to) and move the latent by (sigma_next - sigma) v.
    Returns the final latent and the x0 preview of every step."""
    sig = shifted_sigmas(steps, shift)
    x = np.array(noise, dtype=dtype, copy=True)
    previews = []
    for i in range(steps):
        v = transformer_forward(text, x, refs, segs, io_w, emb_w, w_mod, per_mode, joint, rope,
                                sig[i], t_target=sig[i + 1] if distilled else None, dtype=dtype)
        previews.append(x0_preview(x, v, sig[i]))
        x = euler_step(x, v, sig[i], sig[i + 1])
    return x, previews


# --------------------------------------------------------------------------
# rowwise FP8 ("fp8r") block linears
#   [P1 "Smaller GPUs, single files, and custom LoRA training": the
#   transformer also ships as a rowwise-FP8 single file]; [P4 "What Black
#   Forest Labs released": FP8 files and the GPUs that have FP8 kernels];
#   [P5 architecture notes: fp8r is row-level FP8].
# Readings: the 8-bit format is e4m3 in the OCP 8-bit floating-point form
# (sign, 4 exponent bits with bias 7, 3 mantissa bits; exponent field 15
# with mantissa 7 is NaN, there are no infinities, the largest finite value
# is 448).  A weight matrix [out][in] keeps one scale per output row; the
# input of each quantised linear is quantised the same way per token row
# when the linear runs.  A row with largest magnitude a gets the scale
# s = a / 448 and the codes round(v * (448 / a)), nearest with ties to the
# even code, clamped to +-448; the decision is taken in fp32 (the scale, the
# multiplier and the product are fp32 operations).  An all-zero row gets
# s = 0 and zero codes.  The quantised linears are the block's two fused
# GEMMs: h -> [q | k | v | gate | up] and [o | act] -> out.
# --------------------------------------------------------------------------
E4M3_MAX = 448.0


def e4m3_values():
    """Value of each of the 256 e4m3 codes (NaN for the two NaN codes)."""
    code = np.arange(256)
    sign = np.where(code >> 7, -1.0, 1.0)
    e = (code >> 3) & 15
    m = (code & 7).astype(np.float64)
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * 2.0 ** (e - 7.0))
    val = sign * mag
    val[(e == 15) & (code & 7 == 7)] = np.nan
    return val


E4M3 = e4m3_values()


def e4m3_encode(y):
    """Codes of y rounded to e4m3: nearest value, ties to the even code,
    magnitudes above 448 saturated to 448, the sign kept (also on zero)."""
    y = np.asarray(y, dtype=np.float64)
    a = np.minimum(np.abs(y), E4M3_MAX)
    # spacing of the values around a: 2^(e - 3) in binade [2^e, 2^(e+1)),
    # e >= -6 (below 2^-6 the subnormals keep the spacing 2^-9)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.maximum(e, -6.0)
    step = 2.0 ** (e - 3.0)
    n = np.round(a / step)                     # half to even
    mag = n * step                             # exact: n < 2^5
    # code of the magnitude: field from its binade, mantissa from the step
    ef = np.floor(np.log2(np.where(mag > 0, mag, 1.0)))
    normal = mag >= 2.0 ** -6
    exp_field = np.where(normal, ef + 7.0, 0.0)
    mant = np.where(normal, mag / 2.0 ** ef * 8.0 - 8.0, mag / 2.0 ** -9)
    code = (exp_field.astype(np.int64) << 3) | mant.astype(np.int64)
    code = np.where(np.signbit(y), code | 0x80, code)
    return code.astype(np.uint8)


def quantize_rowwise(a):
    """Rowwise e4m3 quantisation of a 2-D array (read as fp32): returns
    (codes uint8 [R][K], scales fp32 [R]) with a ~= E4M3[codes] * scale."""
    a32 = np.asarray(a, dtype=np.float32)
    amax = np.max(np.abs(a32), axis=1) if a32.shape[1] else np.zeros(a32.shape[0], np.float32)
    pos = amax > 0
    mult = np.zeros_like(amax)
    mult[pos] = np.float32(E4M3_MAX) / amax[pos]
    y = a32 * mult[:, None]                    # fp32 product
    codes = e4m3_encode(y)
    scale = (amax / np.float32(E4M3_MAX)).astype(np.float32)
    return codes, scale


def dequantize_rowwise(codes, scale, dtype=np.float64):
    """E4M3[codes] * scale per row (exact in float64)."""
    return (E4M3[np.asarray(codes)] * np.asarray(scale, np.float64)[:, None]).astype(dtype)


def fake_quantize_rows(a, dtype=np.float64):
    """The values a rowwise-quantised operand stands for."""
    codes, scale = quantize_rowwise(a)
    return dequantize_rowwise(codes, scale, dtype)


def fused_block_matrices(w):
    """The block's two fused linears as plain matrices (bf16 values):
    W1 = [wq; wk; wv; w_gate; w_up] [3D + 2F][D] and W2 = [wo | w_down]
    [D][D + F]."""
    f = _weights(w, np.float64)
    w1 = np.concatenate([f["wq"], f["wk"], f["wv"], f["w_gate"], f["w_up"]], axis=0)
    w2 = np.concatenate([f["wo"], f["w_down"]], axis=1)
    return w1, w2


def quantize_block_weights(w):
    """Rowwise-FP8 form of one block's weights: {"w1": (codes, scales),
    "w2": (codes, scales), "q_norm", "k_norm"} with W1, W2 as in
    fused_block_matrices."""
    w1, w2 = fused_block_matrices(w)
    return {"w1": quantize_rowwise(w1), "w2": quantize_rowwise(w2),
            "q_norm": np.asarray(w["q_norm"]), "k_norm": np.asarray(w["k_norm"])}


def block_forward_quantized(x, w1, w2, norms, segs, mod, rope, act_quant, heads=None,
                            dtype=np.float64, eps_ln=EPS_LN, eps_rms=EPS_RMS, keep=False,
                            rows=None, attn_chunk=None):
    """block_forward with the weights given as the fused W1 [3D + 2F][D] and
    W2 [D][D + F] (any values, e.g. dequantised codes) and with act_quant
    applied to the input of each fused linear, the modulated h and the
    concatenation [o | act].  norms = (q_norm, k_norm).  rows: evaluate the
    output only at these rows (keys and values still come from every
    token).  keep=True also returns {h, y1, o, act, cat, out}."""
    x = np.asarray(x, dtype=dtype)
    n, width = x.shape
    q_norm, k_norm = (as_float(v, dtype) for v in norms)
    hd = q_norm.shape[0]
    if heads is None:
        heads = width // hd
    f = (w1.shape[0] - 3 * width) // 2
    shift, scale, gate = _row_modulation(segs, mod, n, dtype)
    h = modulate(layer_norm(x, eps_ln), shift, scale)
    hq = np.asarray(act_quant(h), dtype=dtype)
    w1 = as_float(w1, dtype)
    k = (hq @ w1[width:2 * width].T).reshape(n, heads, hd)
    v = (hq @ w1[2 * width:3 * width].T).reshape(n, heads, hd)
    k = apply_rope(rms_norm_heads(k, k_norm, eps_rms), rope)
    sel = np.arange(n) if rows is None else np.asarray(rows, dtype=np.int64)
    y1 = hq[sel] @ w1[np.r_[0:width, 3 * width:3 * width + 2 * f]].T
    q = y1[:, :width].reshape(len(sel), heads, hd)
    q = apply_rope(rms_norm_heads(q, q_norm, eps_rms), rope[sel])
    o = attention(q, k, v, chunk=attn_chunk).reshape(len(sel), width)
    act = silu(y1[:, width:width + f]) * y1[:, width + f:]
    cat = np.concatenate([o, act], axis=1)
    out = np.asarray(act_quant(cat), dtype=dtype) @ as_float(w2, dtype).T
    x_new = x[sel] + gate[sel] * out
    if keep:
        return x_new, {"h": h, "y1": y1, "o": o, "act": act, "cat": cat, "out": out}
    return x_new


def block_forward_fp8(x, w8, segs, mod, rope, heads=None, dtype=np.float64, rows=None,
                      keep=False, attn_chunk=None):
    """One block with rowwise-FP8 linears: the weights of
    quantize_block_weights, and h and [o | act] quantised per token row
    (the linear itself is exact on the dequantised values)."""
    w1 = dequantize_rowwise(*w8["w1"])
    w2 = dequantize_rowwise(*w8["w2"])
    return block_forward_quantized(x, w1, w2, (w8["q_norm"], w8["k_norm"]), segs, mod, rope,
                                   fake_quantize_rows, heads=heads, dtype=dtype, rows=rows,
                                   keep=keep, attn_chunk=attn_chunk)
