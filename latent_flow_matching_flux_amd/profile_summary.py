"""Summaries of rocprofv3 output for the block kernels (markdown tables).

    python -m latent_flow_matching_flux_amd.profile_summary trace DIR
    python -m latent_flow_matching_flux_amd.profile_summary pmc DIR [DIR ...]
    python -m latent_flow_matching_flux_amd.profile_summary report TRACE_DIR PMC_DIR ...
    python -m latent_flow_matching_flux_amd.profile_summary traffic FETCH_DIR WRITE_DIR
    python -m latent_flow_matching_flux_amd.profile_summary stack DIR

`trace` reads the *_kernel_trace.csv files under DIR (rocprofv3
--kernel-trace --output-format csv) and gives, per kernel and per grid size,
the launch count, mean / min / max duration and the scratch (private
segment) bytes per lane.  `pmc` reads the *_counter_collection.csv files
under each DIR (rocprofv3 --pmc ...) and gives, per kernel and grid size, the
mean of every counter over the dispatches, plus the derived figures the
counters support:

  MFMA busy   SQ_VALU_MFMA_BUSY_CYCLES / (SIMDs x GRBM_GUI_ACTIVE / 8): share
              of the SIMDs' cycles their matrix unit was busy (the CSV gives
              GRBM_GUI_ACTIVE summed over the 8 XCDs)
  clock       SQ_BUSY_CYCLES / 32 / duration (SQ_BUSY_CYCLES sums the busy
              cycles of the 32 shader engines)
  VALU busy   SQ_ACTIVE_INST_VALU / (CUs x GRBM_GUI_ACTIVE / 8)
  LDS active  SQ_LDS_IDX_ACTIVE / (CUs x GRBM_GUI_ACTIVE / 8): cycles the LDS
              served indexed (ds_*) instructions; the direct global->LDS
              loads are not counted
  DRAM bytes  32 x TCC_EA0_RDREQ_DRAM_32B (reads), 32 x
              TCC_EA0_WRREQ_WRITE_DRAM_32B (writes); FETCH_SIZE / WRITE_SIZE
              are the L2's requests beyond itself (Infinity Cache or DRAM)

`report` combines a trace and counter passes of `bench.py --block-only`
(the joint block at 8432 tokens) into one table per block kernel, with the
algorithmic bytes of each kernel at that size beside the measured ones.

`traffic` turns a FETCH_SIZE pass and a WRITE_SIZE pass of the same
command into the JSON record `bench.py` reports as roofline.traffic (bytes
per gemm_proj dispatch, each counter scaled by what it reads for the block
input's plain device copy of known size), stamped with the sha256 prefix of
the GEMM sources' code (comments and whitespace ignored) so that a record
taken on other kernel code is not used.

`stack` reads the kernel trace of a stack bench (`bench.py --no-block`) and
groups the block kernels' launches by the block call they belong to, in
launch order from the first k_rope_tables launch: a k_ln_modulate opens a
call, the k_gemm_proj grid gives its rows (grid / 108 tiles per 256 rows at
the model dims), and a call with several k_attention launches is a grouped
per-mode call (one attention launch per stream length, in launch order);
calls whose LayerNorm is k_ln_modulate_f8 are the rowwise-FP8 ones.

Kernel names are shortened to the function name (k_gemm_proj, ...).
"""
import csv
import glob
import hashlib
import json
import os
import re
import statistics
import sys
from collections import defaultdict

CUS = 256             # MI355X
SIMDS = 4 * CUS
XCDS = 8
SHADER_ENGINES = 32   # 8 XCDs x 4 shader engines


def short(name):
    m = re.search(r"(k_[a-z0-9_]+)(<(true|false), (true|false)>)?", name)
    if m:
        base = m.group(1)
        t = re.search(r"ILb([01])ELb([01])E", name)   # mangled names
        if t:
            base += f"<{'T' if t.group(1) == '1' else 'F'},{'T' if t.group(2) == '1' else 'F'}>"
        elif m.group(2):
            base += f"<{m.group(3)[0].upper()},{m.group(4)[0].upper()}>"
        return base
    return name.split("(")[0][:48]


def _rows(pattern, d):
    out = []
    for path in sorted(glob.glob(os.path.join(d, "**", pattern), recursive=True)):
        with open(path, newline="") as f:
            out.extend(csv.DictReader(f))
    return out


def _get(row, *keys, default=None):
    for k in keys:
        if k in row and row[k] != "":
            return row[k]
    return default


def _grid(row):
    g = _get(row, "Grid_Size_X", "Grid_Size", default="0")
    wg = _get(row, "Workgroup_Size_X", "Workgroup_Size", default="1")
    try:
        return int(g) // max(int(wg), 1)
    except ValueError:
        return 0


def trace(d):
    rows = _rows("*kernel_trace.csv", d)
    by = defaultdict(list)
    scratch = {}
    for r in rows:
        k = short(r["Kernel_Name"])
        dur = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
        by[(k, _grid(r))].append(dur)
        scratch[k] = max(scratch.get(k, 0), int(_get(r, "Private_Segment_Size", "Scratch_Size",
                                                     default="0")))
    total = sum(sum(v) for v in by.values())
    print("| kernel | workgroups | calls | mean (us) | min (us) | max (us) | share | scratch B/lane |")
    print("|---|---|---|---|---|---|---|---|")
    for (k, g), v in sorted(by.items(), key=lambda kv: -sum(kv[1])):
        print(f"| {k} | {g} | {len(v)} | {statistics.mean(v):.1f} | {min(v):.1f} | {max(v):.1f} "
              f"| {100 * sum(v) / total:.1f}% | {scratch[k]} |")


def pmc(dirs):
    vals = defaultdict(lambda: defaultdict(list))
    durs = defaultdict(list)
    for d in dirs:
        for r in _rows("*counter_collection.csv", d):
            key = (short(r["Kernel_Name"]), _grid(r))
            vals[key][r["Counter_Name"]].append(float(r["Counter_Value"]))
            if "End_Timestamp" in r and r["End_Timestamp"]:
                dur = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
                durs[(key, d)].append(dur)
    for key in sorted(vals):
        k, g = key
        c = {n: statistics.mean(v) for n, v in vals[key].items()}
        n_disp = max(len(v) for v in vals[key].values())
        print(f"\n### {k}, {g} workgroups ({n_disp} dispatches per pass)\n")
        print("| counter | mean per dispatch |")
        print("|---|---|")
        for n in sorted(c):
            print(f"| {n} | {c[n]:.6g} |")
        derived = []
        gui = c.get("GRBM_GUI_ACTIVE", 0.0) / XCDS     # the CSV sums it over the XCDs
        if "SQ_VALU_MFMA_BUSY_CYCLES" in c and gui:
            derived.append(("MFMA busy", f"{100 * c['SQ_VALU_MFMA_BUSY_CYCLES'] / (SIMDS * gui):.1f}% of SIMD cycles"))
        if "SQ_ACTIVE_INST_VALU" in c and gui:
            derived.append(("VALU busy", f"{100 * c['SQ_ACTIVE_INST_VALU'] / (CUS * gui):.1f}%"))
        if "SQ_LDS_IDX_ACTIVE" in c and gui:
            derived.append(("LDS active", f"{100 * c['SQ_LDS_IDX_ACTIVE'] / (CUS * gui):.1f}% of CU cycles"))
        if "SQ_VALU_MFMA_COEXEC_CYCLES" in c and c.get("SQ_VALU_MFMA_BUSY_CYCLES"):
            derived.append(("VALU co-issued with MFMA",
                            f"{100 * c['SQ_VALU_MFMA_COEXEC_CYCLES'] / c['SQ_VALU_MFMA_BUSY_CYCLES']:.1f}% of MFMA-busy cycles"))
        if "SQ_LDS_BANK_CONFLICT" in c and c.get("SQ_ACTIVE_INST_LDS"):
            derived.append(("LDS bank-conflict cycles",
                            f"{100 * c['SQ_LDS_BANK_CONFLICT'] / c['SQ_ACTIVE_INST_LDS']:.2f}% of LDS-active cycles"))
        if "FETCH_SIZE" in c:
            derived.append(("L2 fetch beyond L2", f"{c['FETCH_SIZE'] * 1024 / 1e6:.1f} MB"))
        if "TCC_EA0_RDREQ_DRAM_32B" in c:
            derived.append(("DRAM read", f"{32 * c['TCC_EA0_RDREQ_DRAM_32B'] / 1e6:.1f} MB"))
        if "WRITE_SIZE" in c:
            derived.append(("L2 write beyond L2", f"{c['WRITE_SIZE'] * 1024 / 1e6:.1f} MB"))
        if "TCC_EA0_WRREQ_WRITE_DRAM_32B" in c:
            derived.append(("DRAM write", f"{32 * c['TCC_EA0_WRREQ_WRITE_DRAM_32B'] / 1e6:.1f} MB"))
        for d in dirs:
            if (key, d) in durs and "SQ_BUSY_CYCLES" in c:
                mean_us = statistics.mean(durs[(key, d)])
                derived.append(("clock (SQ_BUSY_CYCLES / engines / duration)",
                                f"{c['SQ_BUSY_CYCLES'] / SHADER_ENGINES / mean_us / 1e3:.2f} GHz "
                                f"over {mean_us:.1f} us"))
                break
        if derived:
            print()
            for n, v in derived:
                print(f"- {n}: {v}")


def _block_kernels(dirs, base_names=False):
    """Mean counter values per dispatch of each kernel's most frequent
    launch shape, merged over the counter passes (keyed by the function
    name alone with base_names)."""
    vals = defaultdict(lambda: defaultdict(list))
    for d in dirs:
        for r in _rows("*counter_collection.csv", d):
            k = short(r["Kernel_Name"])
            if base_names:
                k = k.split("<")[0]
            vals[(k, _grid(r))][r["Counter_Name"]].append(float(r["Counter_Value"]))
    best = {}
    for (k, g), c in vals.items():
        n = max(len(v) for v in c.values())
        if k not in best or n > best[k][1]:
            best[k] = (g, n, {name: statistics.mean(v) for name, v in c.items()})
    return best


def report(trace_dir, pmc_dirs, tokens=8432, D=3072, F=9216, H=24):
    """Markdown table of the block kernels of `bench.py --block-only`."""
    rows = _rows("*kernel_trace.csv", trace_dir)
    dur = defaultdict(list)
    scratch = {}
    for r in rows:
        k = short(r["Kernel_Name"]).split("<")[0]
        dur[k].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
        scratch[k] = max(scratch.get(k, 0), int(_get(r, "Private_Segment_Size", "Scratch_Size",
                                                     default="0")))
    c = _block_kernels(pmc_dirs, base_names=True)
    n_pad = (tokens + 255) // 256 * 256
    mb = 1e6
    alg = {  # algorithmic HBM bytes per launch at this size
        "k_ln_modulate": tokens * D * 4 + n_pad * D * 2,
        "k_gemm_proj": n_pad * D * 2 + (3 * D + 2 * F) * D * 2 + 3 * n_pad * D * 2 + n_pad * F * 2,
        "k_attention": 3 * H * n_pad * 128 * 2 + n_pad * D * 2,
        "k_gemm_out": n_pad * (D + F) * 2 + D * (D + F) * 2 + 2 * tokens * D * 4,
    }
    copy = c.get("__amd_rocclr_copyBuffer")
    fscale = wscale = 1.0
    if copy and copy[2].get("FETCH_SIZE") and copy[2].get("WRITE_SIZE"):
        nbytes = tokens * D * 4
        fscale = nbytes / (copy[2]["FETCH_SIZE"] * 1024)
        wscale = nbytes / (copy[2]["WRITE_SIZE"] * 1024)
    print(f"Calibration: the block's input copy (`__amd_rocclr_copyBuffer`, {tokens * D * 4} B "
          f"read and written) gives FETCH_SIZE x {fscale:.4f} and WRITE_SIZE x {wscale:.4f}; "
          f"32 x TCC_EA0_RDREQ_DRAM_32B reads {32 * copy[2].get('TCC_EA0_RDREQ_DRAM_32B', 0) / mb:.1f} MB "
          f"for it (exact).\n" if copy else "")
    print("| kernel | launches | mean (us) | clock (GHz) | MFMA busy | VALU busy | LDS active | "
          "LDS bank conflicts | L2 fetch beyond L2 (MB) | memory-side reads (MB) | writes (MB) | "
          "algorithmic (MB) | scratch B/lane |")
    print("|" + "---|" * 13)
    for k in ("k_ln_modulate", "k_gemm_proj", "k_attention", "k_attention_fixup", "k_gemm_out",
              "k_gemm_out_fixup"):
        if k not in c:
            continue
        g, n, v = c[k]
        d = dur.get(k, [0.0])
        mean_us = statistics.mean(d)
        gui = v.get("GRBM_GUI_ACTIVE", 0.0) / XCDS     # summed over the XCDs
        clk = v.get("SQ_BUSY_CYCLES", 0.0) / SHADER_ENGINES / (mean_us * 1e3) if mean_us else 0
        mfma = 100 * v.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) / (SIMDS * gui) if gui else 0
        valu = 100 * v.get("SQ_ACTIVE_INST_VALU", 0.0) / (CUS * gui) if gui else 0
        lds = 100 * v.get("SQ_LDS_IDX_ACTIVE", 0.0) / (CUS * gui) if gui else 0
        bank = (100 * v.get("SQ_LDS_BANK_CONFLICT", 0.0) / v["SQ_ACTIVE_INST_LDS"]
                if v.get("SQ_ACTIVE_INST_LDS") else 0)
        fetch = v.get("FETCH_SIZE", 0.0) * 1024 * fscale / mb
        dram = 32 * v.get("TCC_EA0_RDREQ_DRAM_32B", 0.0) / mb
        wr = v.get("WRITE_SIZE", 0.0) * 1024 * wscale / mb
        a = alg.get(k)
        print(f"| {k} | {len(d)} | {mean_us:.1f} | {clk:.2f} | {mfma:.1f}% | {valu:.1f}% | "
              f"{lds:.1f}% | {bank:.2f}% | {fetch:.1f} | {dram:.1f} | {wr:.1f} | "
              f"{a / mb if a else float('nan'):.1f} | {scratch.get(k, 0)} |")


# the sources whose hash stamps a traffic record (bench.py checks the same)
KERNEL_SOURCES = ("gemm.hip", "common.hpp")


def code_text(src):
    """C++ source without comments and with whitespace runs collapsed, so
    that a comment-only edit keeps the hash."""
    src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
    src = re.sub(r"//[^\n]*", " ", src)
    return " ".join(src.split())


def source_hash(read=None):
    """sha256 prefix of the GEMM sources' code (comments ignored); `read`
    maps a file name to its text (default: the working tree)."""
    here = os.path.dirname(os.path.abspath(__file__))
    if read is None:
        def read(name):
            with open(os.path.join(here, "csrc", name)) as f:
                return f.read()
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        h.update(code_text(read(name)).encode())
    return h.hexdigest()[:16]


def traffic(fetch_dir, write_dir, tokens=8432, D=3072, F=9216):
    """JSON record of gemm_proj's HBM-side bytes per dispatch."""
    c = _block_kernels([fetch_dir, write_dir], base_names=True)
    copy = c["__amd_rocclr_copyBuffer"][2]
    g, n, v = c["k_gemm_proj"]
    nbytes = tokens * D * 4
    fscale = nbytes / (copy["FETCH_SIZE"] * 1024)
    wscale = nbytes / (copy["WRITE_SIZE"] * 1024)
    n_pad = (tokens + 255) // 256 * 256
    rec = {
        "kernel": "gemm_proj",
        "workload": f"joint block over the {tokens}-token edit sequence (bench.py --block-only: "
                    f"5 warm-up + 20 timed calls)",
        "tokens": tokens,
        "source_hash": source_hash(),
        "dispatches": n,
        "fetch_kib_mean": v["FETCH_SIZE"],
        "write_kib_mean": v["WRITE_SIZE"],
        "fetch_scale": fscale,
        "write_scale": wscale,
        "bytes_per_launch": v["FETCH_SIZE"] * 1024 * fscale + v["WRITE_SIZE"] * 1024 * wscale,
        "memory_side_read_bytes": 32 * v.get("TCC_EA0_RDREQ_DRAM_32B", 0.0),
        "algorithmic_bytes": float(n_pad * D * 2 + (3 * D + 2 * F) * D * 2 + 3 * n_pad * D * 2
                                   + n_pad * F * 2),
        "commands": [
            f"rocprofv3 --pmc FETCH_SIZE TCC_EA0_RDREQ_DRAM_32B --output-format csv -d {fetch_dir} "
            f"-o pmc3 -- python3 bench.py --block-only",
            f"rocprofv3 --pmc WRITE_SIZE TCC_EA0_WRREQ_WRITE_DRAM_32B --output-format csv -d "
            f"{write_dir} -o pmc4 -- python3 bench.py --block-only",
            f"python -m latent_flow_matching_flux_amd.profile_summary traffic {fetch_dir} {write_dir}"],
    }
    print(json.dumps(rec, indent=1))


BLOCK_KERNELS = ("k_ln_modulate", "k_quant_rows", "k_gemm_proj", "k_attention",
                 "k_attention_fixup", "k_gemm_out", "k_gemm_out_fixup")


def stack(d, n_n=108):
    """Launches of a stack trace by block call (see the module docstring)."""
    rows = sorted(_rows("*kernel_trace.csv", d), key=lambda r: int(r["Start_Timestamp"]))
    start = next((i for i, r in enumerate(rows) if short(r["Kernel_Name"]) == "k_rope_tables"), 0)
    rows = rows[start:]
    by = defaultdict(list)
    scratch = {}
    order = []
    call = []   # the current block call's launches: (kernel, duration)

    def close():
        if not call:
            return
        grid = next((g for k, _, g in call if k.startswith("k_gemm_proj")), 0)
        tokens = grid // n_n * 256
        n_attn = sum(1 for k, _, _ in call if k == "k_attention")
        fp8 = any(k == "k_ln_modulate_f8" for k, _, _ in call)
        label = (("fp8r, " if fp8 else "") + f"{tokens} rows"
                 + (", per-mode (grouped)" if n_attn > 1 else ""))
        a = 0
        for k, dur, _ in call:
            if k == "k_attention" and n_attn > 1:
                a += 1
            key = (k, label + (f", attention launch {a} of {n_attn}"
                               if k.startswith("k_attention") and n_attn > 1 else ""))
            if key not in by:
                order.append(key)
            by[key].append(dur)
        call.clear()

    for r in rows:
        k = short(r["Kernel_Name"])
        dur = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
        scratch[k] = max(scratch.get(k, 0), int(_get(r, "Private_Segment_Size", "Scratch_Size",
                                                     default="0")))
        base = k.split("<")[0]
        if base == "k_ln_modulate" or base == "k_ln_modulate_f8":
            close()
        if base.startswith("k_ln_modulate") or (base in BLOCK_KERNELS and call):
            call.append((k, dur, _grid(r)))
        else:
            close()   # any other launch ends the block call (weight quantisation at load, ...)
            if (k, "-") not in by:
                order.append((k, "-"))
            by[(k, "-")].append(dur)
    close()
    total = sum(sum(v) for v in by.values())
    print("| kernel | block call | launches | mean (us) | min (us) | max (us) | share of GPU time "
          "| scratch B/lane |")
    print("|---|---|---|---|---|---|---|---|")
    for key in order:
        k, label = key
        v = by[key]
        print(f"| {k} | {label} | {len(v)} | {statistics.mean(v):.1f} | {min(v):.1f} | "
              f"{max(v):.1f} | {100 * sum(v) / total:.1f}% | {scratch[k]} |")


if __name__ == "__main__":
    if len(sys.argv) >= 3 and sys.argv[1] == "trace":
        trace(sys.argv[2])
    elif len(sys.argv) >= 3 and sys.argv[1] == "pmc":
        pmc(sys.argv[2:])
    elif len(sys.argv) >= 4 and sys.argv[1] == "report":
        report(sys.argv[2], sys.argv[3:])
    elif len(sys.argv) == 3 and sys.argv[1] == "stack":
        stack(sys.argv[2])
    elif len(sys.argv) == 4 and sys.argv[1] == "traffic":
        traffic(sys.argv[2], sys.argv[3])
    else:
        print(__doc__)
        sys.exit(2)
