"""Summaries of rocprofv3 output for the block kernels (markdown tables).

    python -m latent_flow_matching_flux_amd.profile_summary trace DIR
    python -m latent_flow_matching_flux_amd.profile_summary pmc DIR [DIR ...]
    python -m latent_flow_matching_flux_amd.profile_summary report TRACE_DIR PMC_DIR ...

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

Kernel names are shortened to the function name (k_gemm_proj, ...).
"""
import csv
import glob
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
    m = re.search(r"(k_[a-z0-9_]+)", name)
    if m:
        base = m.group(1)
        t = re.search(r"ILb([01])ELb([01])E", name)
        if t:
            base += f"<{'T' if t.group(1) == '1' else 'F'},{'T' if t.group(2) == '1' else 'F'}>"
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


def _block_kernels(dirs):
    """Mean counter values per dispatch of each kernel's most frequent
    launch shape, merged over the counter passes."""
    vals = defaultdict(lambda: defaultdict(list))
    for d in dirs:
        for r in _rows("*counter_collection.csv", d):
            vals[(short(r["Kernel_Name"]), _grid(r))][r["Counter_Name"]].append(
                float(r["Counter_Value"]))
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
        k = short(r["Kernel_Name"])
        dur[k].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
        scratch[k] = max(scratch.get(k, 0), int(_get(r, "Private_Segment_Size", "Scratch_Size",
                                                     default="0")))
    c = _block_kernels(pmc_dirs)
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


if __name__ == "__main__":
    if len(sys.argv) >= 3 and sys.argv[1] == "trace":
        trace(sys.argv[2])
    elif len(sys.argv) >= 3 and sys.argv[1] == "pmc":
        pmc(sys.argv[2:])
    elif len(sys.argv) >= 4 and sys.argv[1] == "report":
        report(sys.argv[2], sys.argv[3:])
    else:
        print(__doc__)
        sys.exit(2)
