"""Shared helpers for the GPU tests: upload seeded inputs, run the C ABI,
compare with the oracle."""
import numpy as np
import torch

import latent_flow_matching_flux_amd as F
import synth

DEV = "cuda:0"

# parity bar: bf16 compute with fp32 accumulation against the fp32/fp64 oracle
MAXABS_TOL = 3e-2
COS_TOL = 0.9995


def bf16_dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(DEV).view(torch.bfloat16)


def upload_weights(w):
    out = {}
    for k, v in w.items():
        if v.dtype == np.uint16:
            out[k] = bf16_dev(v)
        else:
            out[k] = torch.from_numpy(np.ascontiguousarray(v, np.float32)).to(DEV)
    return out


def rope_dev(layout):
    n = layout.n_tokens
    rope = torch.empty((max(n, 1), 64, 2), dtype=torch.float32, device=DEV)
    F.rope_tables_build(layout, rope, n_tokens=n)
    return rope[:n] if n else rope[:0]


def workspace(dims, n):
    nbytes = F.workspace_bytes(dims, n)
    return torch.empty(max(nbytes, 256), dtype=torch.uint8, device=DEV)


def metrics(got, want):
    got = np.asarray(got, np.float64).ravel()
    want = np.asarray(want, np.float64).ravel()
    maxabs = float(np.max(np.abs(got - want))) if got.size else 0.0
    denom = np.linalg.norm(got) * np.linalg.norm(want)
    cos = float(got @ want / denom) if denom > 0 else 1.0
    return maxabs, cos


def assert_close(got, want, what, maxabs_tol=MAXABS_TOL, cos_tol=COS_TOL):
    """One block's fp32 output against the oracle: max-abs and cosine."""
    maxabs, cos = metrics(got, want)
    print(f"[parity] {what}: max-abs {maxabs:.3e} (tol {maxabs_tol:.3e}) cosine {cos:.8f}")
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    assert maxabs <= maxabs_tol and cos >= cos_tol, \
        f"{what}: max-abs {maxabs:.3e} (tol {maxabs_tol}), cosine {cos:.7f} (tol {cos_tol})"
    return maxabs, cos


# A bf16-stored intermediate carries its own rounding (half an ulp, 2^-9
# relative) on top of the operand rounding upstream of it; elementwise bound
# |got - want| <= 3e-2 + 2^-7 |want| (two bf16 ulps relative).
BF16_REL = 2.0 ** -7


def assert_close_bf16(got, want, what, cos_tol=COS_TOL):
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    err = np.abs(got - want)
    bound = MAXABS_TOL + BF16_REL * np.abs(want)
    worst = float(np.max(err / bound)) if err.size else 0.0
    _, cos = metrics(got, want)
    print(f"[parity] {what}: max-abs {err.max():.3e}, worst err/bound {worst:.3f}, cosine {cos:.8f}")
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    assert worst <= 1.0 and cos >= cos_tol, f"{what}: err/bound {worst:.3f}, cosine {cos:.7f}"


def assert_close_stack(got, want, x_in, what):
    """Stack output: bf16 rounding is relative, so over many blocks the
    absolute bound scales with the residual stream: max-abs <= 3e-2 * max(1,
    rms(want)); cosine >= 0.9995 on x_out and on x_out - x_in."""
    rms = float(np.sqrt(np.mean(np.asarray(want, np.float64) ** 2)))
    tol = MAXABS_TOL * max(1.0, rms)
    assert_close(got, want, what + " x_out", maxabs_tol=tol)
    dw = np.asarray(want, np.float64) - x_in
    assert_close(np.asarray(got, np.float64) - x_in, dw, what + " delta", maxabs_tol=tol)


def seg_tuples(segs):
    return [(s.start, s.count, s.mode) for s in segs]


def bf16_to_np(t):
    return t.float().cpu().numpy()


def vt_unpermute(vt, n):
    """Undo the key permutation of the transposed value store: returns
    [H][128][n] in token order."""
    H, d, n_pad = vt.shape
    idx = np.arange(n_pad)
    g = (idx >> 2) & 3
    gp = ((g & 1) << 1) | (g >> 1)
    pos = (idx & ~15) | (gp << 2) | (idx & 3)
    return vt[:, :, pos][:, :, :n]
