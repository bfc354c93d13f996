#!/usr/bin/env python3
"""Throughput of the FLUX.3 Image Klein block stack on one MI355X.

One step is the whole hot path over one batch: the rotary tables for the
token layout, the two stages' modulation vectors from the timesteps (image
t drawn U(0, 1) with seed 0, text and reference t = 0), then the two-stage
stack -- 5 per-mode blocks on each stream (text, noisy image, reference;
each stream attends only to itself) and 28 joint blocks over the
concatenated sequence -- on the single-reference edit workload [240 text |
64x64 image | 64x64 reference] = 8432 tokens at width 3072, 24 heads x 128,
SwiGLU hidden 9216, bf16 operands with fp32 accumulation and an fp32
residual stream.  Weights (43 distinct blocks, the timestep embedder and
6 modulation linears) are seeded random N(0, 0.02^2) in bf16, tokens
N(0, 1); everything is resident in HBM before timing starts.  The block
matrices are copied once, at load, into the GEMMs' packed operand layout
(flux3_weights_pack; --linear-weights keeps torch's Linear layout).

value = block-token passes per second = (5 + 28) * 8432 / step time, the
rate at which tokens go through transformer blocks.  Per-kernel durations
come from HIP events the library records around each of its launches on the
launch stream, inside the timed region.

The JSON line also carries the single joint block at 8432 tokens, timed
apart from the step loop: 5 warm-up and 20 timed calls, each bracketed by
HIP events on the launch stream, rotating 4 weight copies (980 MB) so that
no call finds its weights in the 256 MB Infinity Cache; median and minimum,
block tokens/s = N / t_block, and GEMM / attention TFLOP/s from the
library's per-kernel events over those calls.  "whole_call" times one
flux3_transformer_forward (input linears from 20,480-value text vectors and
128-value latent tokens, both stages' modulation, the 5+28 blocks, the
output layer) and one 16-step distilled flux3_sample over the same blocks.  Peak: the 2516.6 TFLOP/s of
AMD's MI355X spec, next to CUs x clock x 4096 from the device query.

"graph" replays the same step recorded once as a HIP graph (torch.cuda.graph
over the library's launches): the same kernels without the host's launch
gaps, its result checked bit for bit against the eager step.

"fp8r" repeats the joint block and the step loop with the blocks' weights in
the rowwise-FP8 form (flux3_weights_quantize_fp8r: e4m3 codes, one scale per
output row; the GEMM inputs quantised per token inside each block), its GEMM
rates against the 5033 TFLOP/s dense fp8 MFMA peak.  The headline value
stays the bf16 stack.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6      # 256 CU x 2.4 GHz x 4096 dense bf16 FLOP/clk/CU
PEAK_FP8_TFLOPS = 5033.2       # 256 CU x 2.4 GHz x 8192 dense fp8 FLOP/clk/CU
PEAK_HBM_GBS = 8000.0
N_PM, N_JOINT = 5, 28
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemm_proj_edit8432_traffic.json")


def gemm_flops_per_token(d):
    proj = 2 * d.width * (3 * d.width + 2 * d.mlp_hidden)
    out = 2 * (d.width + d.mlp_hidden) * d.width
    return proj, out


def measured_traffic(launch_tokens):
    """HBM bytes per gemm_proj launch from the committed rocprofv3 counter
    summary, or None if absent or taken on a different kernel source."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    from latent_flow_matching_flux_amd.profile_summary import source_hash
    if t.get("source_hash") != source_hash() or t.get("tokens") != launch_tokens:
        return None
    return t.get("bytes_per_launch")


def time_joint_block(F, dims, lay, segs, n, rand, rand_block, reps=20, warmup=5, copies=4,
                     peak=PEAK_BF16_TFLOPS):
    """One joint block over all n tokens: median/min of `reps` event-timed
    calls with rotating weight copies, plus per-kernel GEMM and attention
    rates over the same calls."""
    import statistics
    import torch
    dev = torch.device("cuda:0")
    D = dims.width
    blocks = [rand_block() for _ in range(copies)]
    x0 = rand(n, D, dtype=torch.float32)
    x = torch.empty_like(x0)
    mod = rand(len(segs), 3, D, std=0.07, dtype=torch.float32)
    rope = torch.empty((n, 64, 2), dtype=torch.float32, device=dev)
    F.rope_tables_build(lay, rope)
    ws = torch.empty(F.workspace_bytes(dims, n), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    for i in range(warmup):
        x.copy_(x0)
        F.block_forward(dims, blocks[i % copies], x, segs, mod, rope, ws, stream=stream)
    torch.cuda.synchronize()
    F.profile_reset()
    F.profile_enable(True)
    events = []
    for i in range(reps):
        x.copy_(x0)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        F.block_forward(dims, blocks[i % copies], x, segs, mod, rope, ws, stream=stream)
        e1.record(stream)
        events.append((e0, e1))
    torch.cuda.synchronize()
    F.profile_enable(False)
    stats = {k: F.profile_read(k) for k in F.KERNELS}
    F.profile_reset()
    assert torch.isfinite(x).all(), "non-finite block output"
    ms = sorted(a.elapsed_time(b) for a, b in events)
    proj_fpt, out_fpt = gemm_flops_per_token(dims)
    gemm_flops = (proj_fpt + out_fpt) * n * reps
    attn_flops = 4.0 * D * n * n * reps
    gemm_ms = stats["gemm_proj"]["total_ms"] + stats["gemm_out"]["total_ms"]
    attn_ms = stats["attention"]["total_ms"]
    block_flops = (proj_fpt + out_fpt) * n + 4.0 * D * n * n
    med = statistics.median(ms)
    return {"tokens": n, "reps": reps, "warmup": warmup, "weight_copies": copies,
            "median_ms": med, "min_ms": ms[0],
            "tokens_per_s": n / (med * 1e-3),
            "tflops": block_flops / (med * 1e-3) / 1e12,
            "frac_peak": block_flops / (med * 1e-3) / 1e12 / peak,
            "gemm_tflops": gemm_flops / (gemm_ms * 1e-3) / 1e12,
            "attention_tflops": attn_flops / (attn_ms * 1e-3) / 1e12,
            "kernel_ms": {k: v["total_ms"] / reps for k, v in stats.items()}}


def time_whole_calls(F, dims, lay, segs, n, rand, per_mode, joint, emb_w, mod_w, steps=16,
                     reps=3):
    """One whole transformer call (input linears, both stages' modulation,
    the stack, the output layer) and one full denoise loop of `steps`
    distilled steps, on the same workload and blocks: event-timed, mean of
    `reps` calls after one warm-up, and one loop after a warm-up loop."""
    import torch
    import synth
    dev = torch.device("cuda:0")
    D = dims.width
    TD, LD = synth.TEXT_DIM, synth.LATENT_DIM
    n_text = sum(s.count for s in segs if s.mode == 0)
    n_img = sum(s.count for s in segs if s.mode == 1)
    n_ref = sum(s.count for s in segs if s.mode == 2)
    io = {"w_text": rand(D, TD, std=0.02), "w_img_in": rand(D, LD, std=0.02),
          "w_ref_in": rand(D, LD, std=0.02), "w_final": rand(2 * D, D, std=0.02),
          "w_out": rand(LD, D, std=0.02)}
    tgt = {"w1_tgt": rand(D, 256, std=0.02), "w2_tgt": rand(D, D, std=0.02)}
    mw = [dict(m, **tgt) for m in mod_w]
    text = rand(n_text, TD) if n_text else None
    image = rand(n_img, LD, dtype=torch.float32)
    refs = rand(n_ref, LD, dtype=torch.float32) if n_ref else None
    rope = torch.empty((n, 64, 2), dtype=torch.float32, device=dev)
    F.rope_tables_build(lay, rope)
    io_dims = F.IoDims(TD, LD)
    vel = torch.empty((n_img, LD), dtype=torch.float32, device=dev)
    ws = torch.empty(F.sample_workspace_bytes(dims, io_dims, n), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def call():
        F.transformer_forward(dims, io_dims, io, mw, per_mode, joint, text, image, refs, segs,
                              0.75, rope, vel, ws, t_target=0.7, stream=stream)

    call()
    torch.cuda.synchronize()
    F.profile_reset()
    F.profile_enable(True)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        call()
    e1.record(stream)
    torch.cuda.synchronize()
    F.profile_enable(False)
    io_stats = F.profile_read("io_linears")
    F.profile_reset()
    call_ms = e0.elapsed_time(e1) / reps
    assert torch.isfinite(vel).all(), "non-finite velocity"
    lat = torch.empty_like(image)

    def loop():
        lat.copy_(image)
        F.sample(dims, io_dims, io, mw, per_mode, joint, text, lat, refs, segs, steps, rope, ws,
                 stream=stream)

    loop()
    torch.cuda.synchronize()
    e0.record(stream)
    loop()
    e1.record(stream)
    torch.cuda.synchronize()
    loop_ms = e0.elapsed_time(e1)
    assert torch.isfinite(lat).all(), "non-finite latent"
    return {"transformer_call_ms": call_ms, "transformer_call_tokens_per_s": n / (call_ms * 1e-3),
            "io_linears_ms_per_call": io_stats["total_ms"] / reps,
            "sample_steps": steps, "sample_ms": loop_ms,
            "images_per_s": 1e3 / loop_ms, "reps": reps,
            "what": "transformer call = text/image/reference input linears + both stages' "
                    "modulation from (t, t_target) + 5+28 blocks + output layer; sample = "
                    f"{steps} distilled steps (call + Euler step each), shift 6.93"}


def time_graph_steps(torch, step, x, steps, passes, eager_ms):
    """The step captured once as a HIP graph and replayed `steps` times: the
    same kernels without the host's launch gaps.  The replayed result must
    equal the eager step's bit for bit."""
    want = x.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    g.replay()
    torch.cuda.synchronize()
    assert torch.equal(x, want), "graph replay differs from the eager step"
    t0 = time.perf_counter()
    for _ in range(steps):
        g.replay()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms = (t1 - t0) / steps * 1e3
    del g
    return {"ms_per_step": ms, "block_tokens_per_s": passes / (ms * 1e-3),
            "eager_over_graph": eager_ms / ms,
            "what": "the same step (rope tables, both stages' modulation, x restore, 5+28 "
                    "blocks) recorded once with torch.cuda.graph and replayed"}


def cpu_baseline(workload_name, blocks=5):
    """The oracle, as it stands, on `blocks` joint blocks of the same
    workload: NumPy float32 with the BLAS library and the oracle's attention
    threads on the process's CPU share (at most 16 cores); value in block
    tokens/s."""
    import numpy as np
    import synth
    from oracle import flux3_oracle as O
    wl = synth.workload(workload_name)
    lay = wl.layout
    n = lay.n_tokens
    segs = [(s.start, s.count, s.mode) for s in lay.segments()]
    cores = max(1, min(16, len(os.sched_getaffinity(0))))
    O.THREADS = cores
    w = synth.block_weights(0, 0, synth.DIMS)
    x = synth.tokens(0, n, synth.DIMS.width)
    mod = synth.modulation(0, 0, len(segs), synth.DIMS.width)
    rope = O.rope_tables(O.token_positions(lay.n_text, lay.grid_h, lay.grid_w, lay.refs))
    from threadpoolctl import threadpool_limits
    with threadpool_limits(limits=cores, user_api="blas"):
        t0 = time.perf_counter()
        for _ in range(blocks):
            x = O.block_forward(x, w, segs, mod, rope, dtype=np.float32, attn_chunk=2048)
        dt = time.perf_counter() - t0
    assert np.isfinite(x).all()
    model = "unknown CPU"
    try:
        with open("/proc/cpuinfo") as f:
            model = next(l.split(":", 1)[1].strip() for l in f if l.startswith("model name"))
    except (OSError, StopIteration):
        pass
    return {"value": blocks * n / dt, "unit": "block tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"{blocks} joint blocks over the {n}-token {workload_name} sequence, "
                      f"NumPy float32 ({cores} BLAS and attention threads on {model}), "
                      f"{dt:.1f} s"}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="edit8432")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--linear-weights", action="store_true",
                    help="keep the weights in Linear layout instead of packing them at load")
    ap.add_argument("--no-sample", action="store_true",
                    help="skip the whole-call and denoise-loop timings")
    ap.add_argument("--no-fp8", action="store_true",
                    help="skip the rowwise-FP8 block and step timings")
    ap.add_argument("--no-block", action="store_true",
                    help="skip the single-block, whole-call and denoise-loop timings "
                         "(profiling runs of the step alone)")
    ap.add_argument("--block-only", action="store_true",
                    help="time the single joint block alone and print its figures "
                         "(counter runs of the block kernels at one size)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path; run with --gpus 1",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import latent_flow_matching_flux_amd as F
    import synth

    F.load()
    dev = torch.device("cuda:0")
    dims = synth.DIMS
    wl = synth.workload(args.workload)
    lay = wl.layout
    segs = lay.segments()
    n = lay.n_tokens
    D, Fh = dims.width, dims.mlp_hidden

    g = torch.Generator(device=dev)
    g.manual_seed(0)

    def rand(*shape, std=1.0, dtype=torch.bfloat16):
        return (torch.randn(*shape, generator=g, device=dev, dtype=torch.float32) * std).to(dtype)

    def rand_block(fp8=False):
        w = {"wq": rand(D, D, std=0.02), "wk": rand(D, D, std=0.02), "wv": rand(D, D, std=0.02),
             "wo": rand(D, D, std=0.02), "w_gate": rand(Fh, D, std=0.02),
             "w_up": rand(Fh, D, std=0.02), "w_down": rand(D, Fh, std=0.02),
             "q_norm": torch.ones(128, device=dev), "k_norm": torch.ones(128, device=dev)}
        if fp8:
            # rowwise e4m3 codes and scales, quantised once at load
            buf = torch.empty(F.weights_fp8r_bytes(dims), dtype=torch.uint8, device=dev)
            return F.weights_quantize_fp8r(dims, w, buf)
        if args.linear_weights:
            return w
        # static weights go to the GEMMs' packed operand layout once, at load
        buf = torch.empty(F.weights_packed_bytes(dims), dtype=torch.uint8, device=dev)
        return F.weights_pack(dims, w, buf)

    if args.block_only:
        block = time_joint_block(F, dims, lay, segs, n, rand, rand_block)
        print(json.dumps({"workload": args.workload, "block": block}))
        return

    modes = sorted({s.mode for s in segs})
    per_mode = {m: [rand_block() for _ in range(N_PM)] for m in modes}
    joint = [rand_block() for _ in range(N_JOINT)]
    x0 = rand(n, D, dtype=torch.float32)
    x = torch.empty_like(x0)
    # timestep path: one embedder, a modulation linear per (stage, mode)
    emb_w = {"w1": rand(D, 256, std=0.02), "w2": rand(D, D, std=0.02)}
    mod_w = [dict(emb_w, w_mod={m: rand(3 * D, D, std=0.02) for m in modes}) for _ in range(2)]
    import numpy as np
    t_image = float(np.random.default_rng(0).uniform())
    t_by_mode = (0.0, t_image, 0.0)
    m1 = torch.empty((len(segs), 3, D), dtype=torch.float32, device=dev)
    m2 = torch.empty_like(m1)
    mws = torch.empty(F.modulation_workspace_bytes(dims), dtype=torch.uint8, device=dev)
    rope = torch.empty((n, 64, 2), dtype=torch.float32, device=dev)
    ws = torch.empty(F.workspace_bytes(dims, n), dtype=torch.uint8, device=dev)

    def step(pm=per_mode, jt=joint):
        # on the current stream: the launch stream, or the capture stream
        # while the step is recorded as a graph
        s = torch.cuda.current_stream()
        F.rope_tables_build(lay, rope, stream=s)
        F.modulation_forward(dims, mod_w[0], t_by_mode, segs, m1, mws, stream=s)
        F.modulation_forward(dims, mod_w[1], t_by_mode, segs, m2, mws, stream=s)
        x.copy_(x0)
        F.stack_forward(dims, pm, jt, x, segs, m1, m2, rope, ws, stream=s)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    assert torch.isfinite(x).all(), "non-finite stack output"

    F.profile_reset()
    F.profile_enable(True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    F.profile_enable(False)
    stats = {k: F.profile_read(k) for k in F.KERNELS}
    # the launches over all n tokens (the joint blocks; for the GEMMs also the
    # per-mode blocks, whose streams share one launch per block) apart from
    # the per-stream attention launches
    joint_stats = {k: F.profile_read(k, n_tokens=n) for k in ("gemm_proj", "attention", "gemm_out")}
    F.profile_reset()

    ms_per_step = (t1 - t0) / args.steps * 1e3
    passes = (N_PM + N_JOINT) * n
    graph = time_graph_steps(torch, step, x, args.steps, passes, ms_per_step)
    value = passes / (ms_per_step / 1e3)
    proj_fpt, out_fpt = gemm_flops_per_token(dims)

    def tflops(flops, ms):
        return flops / (ms * 1e-3) / 1e12 if ms > 0 else 0.0

    kern = {}
    for k, st in stats.items():
        ms = st["total_ms"]
        entry = {"launches": st["launches"], "ms_per_step": ms / args.steps,
                 "avg_us": 1e3 * ms / max(st["launches"], 1)}
        if k == "gemm_proj":
            entry["tflops"] = tflops(proj_fpt * st["tokens"], ms)
        elif k == "gemm_out":
            entry["tflops"] = tflops(out_fpt * st["tokens"], ms)
        elif k == "attention":
            entry["tflops"] = tflops(4.0 * D * st["tokens_sq"], ms)
        elif k == "ln_modulate":
            entry["gbs"] = 6.0 * D * st["tokens"] / (ms * 1e-3) / 1e9 if ms > 0 else 0.0
        elif k == "rope_tables":
            entry["gbs"] = 512.0 * st["tokens"] / (ms * 1e-3) / 1e9 if ms > 0 else 0.0
        elif k == "modulation":
            # weights read once per call: embedder + one linear per used mode
            wbytes = 2.0 * (D * 256 + D * D + len(modes) * 3 * D * D)
            entry["gbs"] = wbytes * st["launches"] / (ms * 1e-3) / 1e9 if ms > 0 else 0.0
        if "tflops" in entry:
            entry["frac_peak"] = entry["tflops"] / PEAK_BF16_TFLOPS
        kern[k] = entry

    step_flops = 0.0
    step_flops += proj_fpt * stats["gemm_proj"]["tokens"] + out_fpt * stats["gemm_out"]["tokens"]
    step_flops += 4.0 * D * stats["attention"]["tokens_sq"]
    step_flops /= args.steps

    # dominant kernel: the projection GEMM (the largest FLOP share), over
    # its launches at the full n tokens (each step's 28 joint blocks and 5
    # grouped per-mode blocks); the mean over every launch is given beside it
    gp = joint_stats["gemm_proj"]
    avg_ms = gp["total_ms"] / max(gp["launches"], 1)
    achieved = proj_fpt * n / (avg_ms * 1e-3) / 1e12 if avg_ms > 0 else 0.0
    ga = stats["gemm_proj"]
    all_avg_ms = ga["total_ms"] / max(ga["launches"], 1)
    all_achieved = (proj_fpt * ga["tokens"] / max(ga["launches"], 1) / (all_avg_ms * 1e-3) / 1e12
                    if all_avg_ms > 0 else 0.0)
    roofline = {"bound": "mfma", "kernel": "gemm_proj", "achieved": achieved,
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_TFLOPS,
                "traffic": measured_traffic(n),
                "launches": gp["launches"], "avg_us": 1e3 * avg_ms,
                "work_per_launch": f"{proj_fpt / 1e6:.2f} MFLOP/token x {n} tokens "
                                   f"(the launches over all tokens in the timed steps)",
                "all_launches": {"launches": ga["launches"], "avg_us": 1e3 * all_avg_ms,
                                 "mean_tokens": ga["tokens"] / max(ga["launches"], 1),
                                 "achieved": all_achieved,
                                 "frac": all_achieved / PEAK_BF16_TFLOPS}}
    joint_rates = {}
    for k, st in joint_stats.items():
        ms = st["total_ms"] / max(st["launches"], 1)
        fl = (proj_fpt * n if k == "gemm_proj" else out_fpt * n if k == "gemm_out"
              else 4.0 * D * n * n)
        joint_rates[k] = {"launches": st["launches"], "avg_us": 1e3 * ms,
                    "tflops": tflops(fl, ms), "frac_peak": tflops(fl, ms) / PEAK_BF16_TFLOPS}

    # single joint block over all tokens (the same segments and layout), and
    # the whole transformer call and denoise loop around the same blocks
    block = whole = None
    if not args.no_block:
        block = time_joint_block(F, dims, lay, segs, n, rand, rand_block)
        block["gemm_frac_peak"] = block["gemm_tflops"] / PEAK_BF16_TFLOPS
        block["attention_frac_peak"] = block["attention_tflops"] / PEAK_BF16_TFLOPS
        if not args.no_sample:
            whole = time_whole_calls(F, dims, lay, segs, n, rand, per_mode, joint, emb_w, mod_w)
    fp8 = None
    if not args.no_fp8:
        fp8 = {"weights": "rowwise e4m3 codes + fp32 row scales (flux3_weights_quantize_fp8r); "
                          "h and [o | act] quantised per token in each block",
               "peak_tflops": PEAK_FP8_TFLOPS}
        if not args.no_block:
            b8 = time_joint_block(F, dims, lay, segs, n, rand, lambda: rand_block(True),
                                  peak=PEAK_FP8_TFLOPS)
            b8["gemm_frac_fp8_peak"] = b8["gemm_tflops"] / PEAK_FP8_TFLOPS
            b8["attention_frac_bf16_peak"] = b8["attention_tflops"] / PEAK_BF16_TFLOPS
            fp8["block"] = b8
        pm8 = {m: [rand_block(True) for _ in range(N_PM)] for m in modes}
        jt8 = [rand_block(True) for _ in range(N_JOINT)]
        for _ in range(args.warmup):
            step(pm8, jt8)
        torch.cuda.synchronize()
        assert torch.isfinite(x).all(), "non-finite fp8 stack output"
        F.profile_reset()
        F.profile_enable(True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            step(pm8, jt8)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        F.profile_enable(False)
        st8 = {k: F.profile_read(k) for k in F.KERNELS}
        F.profile_reset()
        ms8 = (t1 - t0) / args.steps * 1e3
        fp8["ms_per_step"] = ms8
        fp8["block_tokens_per_s"] = passes / (ms8 / 1e3)
        fp8["speedup_vs_bf16_step"] = ms_per_step / ms8
        fp8["kernel_ms_per_step"] = {k: v["total_ms"] / args.steps for k, v in st8.items()
                                     if v["launches"]}
        g8 = st8["gemm_proj"]
        g8_ms = g8["total_ms"] / max(g8["launches"], 1)
        g8_tf = proj_fpt * g8["tokens"] / max(g8["launches"], 1) / (g8_ms * 1e-3) / 1e12
        fp8["gemm_proj"] = {"avg_us": 1e3 * g8_ms, "tflops": g8_tf,
                            "frac_fp8_peak": g8_tf / PEAK_FP8_TFLOPS}
        o8 = st8["gemm_out"]
        o8_ms = o8["total_ms"] / max(o8["launches"], 1)
        o8_tf = out_fpt * o8["tokens"] / max(o8["launches"], 1) / (o8_ms * 1e-3) / 1e12
        fp8["gemm_out"] = {"avg_us": 1e3 * o8_ms, "tflops": o8_tf,
                           "frac_fp8_peak": o8_tf / PEAK_FP8_TFLOPS}
        del pm8, jt8
    devinfo = F.device_query(0)
    peak = {"spec_tflops": PEAK_BF16_TFLOPS, "derived_tflops": devinfo["bf16_dense_tflops"],
            "compute_units": devinfo["compute_units"], "clock_mhz": devinfo["clock_khz"] / 1e3,
            "arch": devinfo["arch"], "rule": "CUs x clock x 4096 FLOP/clk (dense bf16 MFMA)"}

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(args.workload)

    out = {
        "metric": "block tokens/s + attn/GEMM TFLOP/s (% bf16 MFMA peak) at 8432 tokens",
        "value": value,
        "unit": "block tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{args.workload}: {wl.description}; rope tables + 2 stages' "
                               f"modulation from t + {N_PM} per-mode blocks per stream + "
                               f"{N_JOINT} joint blocks",
                   "tokens": n, "width": D, "heads": dims.heads, "head_dim": dims.head_dim,
                   "mlp_hidden": Fh, "segments": [[s.start, s.count, s.mode] for s in segs],
                   "t_image": t_image, "t_text": 0.0, "t_reference": 0.0,
                   "weight_layout": "linear" if args.linear_weights else
                   "packed once at load (flux3_weights_pack)"},
        "step_tflops": step_flops / (ms_per_step * 1e-3) / 1e12,
        "step_frac_peak": step_flops / (ms_per_step * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
        "stack_tokens_per_s": n / (ms_per_step / 1e3),
        "kernels": kern,
        "joint_launches": joint_rates,
        "block": block,
        "whole_call": whole,
        "peak": peak,
        "roofline": roofline,
        "graph": graph,
        "fp8r": fp8,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out))


if __name__ == "__main__":
    main()
