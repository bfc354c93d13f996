"""The block and the two-stage stack with bf16 rounding at the GPU path's
storage points -- a tolerance-floor diagnostic for the tests.

NOT a reference and not part of the oracle.  It takes the oracle's steps
(the block of the Diffusers release post's model walk-through, everytik.com
translation; the stage structure of "Speed, architecture, and how the tokens
move", 15jq.com post) in float32 and rounds to bfloat16 (nearest, ties to
even) exactly where the HIP kernels keep a value in bf16:

  h    the modulated LayerNorm output (the projection GEMM's input)
  q, k after RMS normalisation and the rotation (the attention inputs)
  v    the value projection
  P    the softmax numerators before the P.V product (the running sum adds
       them unrounded, in fp32, as the attention kernel does)
  o    the normalised attention output
  act  silu(gate) * up (the output GEMM's second input)

Weights are the same bf16 values as everywhere else; products accumulate in
fp32 and the residual stream stays fp32.  What this shows is how far any
computation that stores these values in bf16 must land from the fp32
oracle, with no other error at all: the floor under the GPU's distance.
Torch CPU operations only; nothing here touches the HIP path.
"""
import numpy as np
import torch

from oracle import flux3_oracle as O


def _bf(t):
    return t.to(torch.bfloat16).to(torch.float32)


def _f32(a):
    return torch.from_numpy(np.ascontiguousarray(O.as_float(a, np.float32)))


def _weights(w):
    return {k: _f32(v) for k, v in w.items()}


def block(x, w, segs, mod, rope, eps=1e-6):
    """One block on fp32 torch x [N][D]; w as the oracle takes it (bf16 bits
    or floats); segs (start, count, mode); mod [n_segs][3][D]; rope
    [N][64][2] fp32 (numpy or torch)."""
    wf = w if isinstance(w.get("wq"), torch.Tensor) else _weights(w)
    n, D = x.shape
    hd = wf["q_norm"].shape[0]
    H = D // hd
    mod = torch.as_tensor(np.asarray(mod, np.float32))
    shift = torch.empty(n, D)
    scale = torch.empty(n, D)
    gate = torch.empty(n, D)
    for s, (start, count, _m) in enumerate(segs):
        shift[start:start + count] = mod[s, 0]
        scale[start:start + count] = mod[s, 1]
        gate[start:start + count] = mod[s, 2]
    rope = torch.as_tensor(np.asarray(rope, np.float32))
    cos, sin = rope[:, None, :, 0], rope[:, None, :, 1]

    mu = x.mean(-1, keepdim=True)
    var = ((x - mu) ** 2).mean(-1, keepdim=True)
    h = _bf((1.0 + scale) * ((x - mu) / torch.sqrt(var + eps)) + shift)

    def qk(wm, nw):
        t = (h @ wm.T).reshape(n, H, hd)
        t = t / torch.sqrt((t * t).mean(-1, keepdim=True) + eps) * nw
        t0, t1 = t[..., 0::2], t[..., 1::2]
        r = torch.empty_like(t)
        r[..., 0::2] = t0 * cos - t1 * sin
        r[..., 1::2] = t0 * sin + t1 * cos
        return _bf(r)

    q = qk(wf["wq"], wf["q_norm"])
    k = qk(wf["wk"], wf["k_norm"])
    v = _bf(h @ wf["wv"].T).reshape(n, H, hd)
    o = torch.empty(n, H, hd)
    sc = 1.0 / np.sqrt(hd)
    for hh in range(H):
        s = (q[:, hh] @ k[:, hh].T) * sc
        p = torch.exp(s - s.max(-1, keepdim=True).values)
        o[:, hh] = (_bf(p) @ v[:, hh]) / p.sum(-1, keepdim=True)
    o = _bf(o.reshape(n, D))
    g = h @ wf["w_gate"].T
    act = _bf(g * torch.sigmoid(g) * (h @ wf["w_up"].T))
    out = o @ wf["wo"].T + act @ wf["w_down"].T
    return x + gate * out


def stack(x, per_mode, joint, segs, mod_stage1, mod_stage2, rope):
    """The oracle's stack composition (stage 1 per segment on its own rows,
    stage 2 over all rows) with the emulated block; shared modulation per
    stage.  Returns float32 numpy."""
    torch.set_num_threads(max(1, torch.get_num_threads()))
    cache = {}

    def wf(w):
        key = id(w)
        if key not in cache:
            cache[key] = _weights(w)
        return cache[key]

    rope = np.asarray(rope, np.float32)
    out = torch.from_numpy(np.array(x, np.float32, copy=True))
    with torch.no_grad():
        for s, (start, count, mode) in enumerate(segs):
            for wb in per_mode.get(mode, []):
                out[start:start + count] = block(out[start:start + count], wf(wb),
                                                 [(0, count, mode)],
                                                 np.asarray(mod_stage1)[s:s + 1],
                                                 rope[start:start + count])
        for wb in joint:
            out = block(out, wf(wb), segs, mod_stage2, rope)
    return out.numpy()
