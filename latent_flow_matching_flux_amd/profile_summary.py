"""Summaries of rocprofv3 output for the block kernels (markdown tables).

    python -m latent_flow_matching_flux_amd.profile_summary trace DIR
    python -m latent_flow_matching_flux_amd.profile_summary pmc DIR [DIR ...]

`trace` reads the *_kernel_trace.csv files under DIR (rocprofv3
--kernel-trace --output-format csv) and gives, per kernel and per grid size,
the launch count, mean / min / max duration and the scratch (private
segment) bytes per lane.  `pmc` reads the *_counter_collection.csv files
under each DIR (rocprofv3 --pmc ...) and gives, per kernel and grid size, the
mean of every counter over the dispatches, plus the derived figures the
counters support:

  MFMA busy   SQ_VALU_MFMA_BUSY_CYCLES / (SIMDs x GRBM_GUI_ACTIVE): share of
              the SIMDs' cycles their matrix unit was busy
  clock       SQ_BUSY_CYCLES / duration (SQ_BUSY_CYCLES counts each shader
              engine's busy cycles; divided by the engine count)
  VALU busy   SQ_ACTIVE_INST_VALU / (4 x SQ_BUSY_CU_CYCLES)
  LDS bytes   SQ_INSTS_LDS is per wave; bandwidth needs the kernel's own
              bytes per instruction, so only counts are reported
  DRAM bytes  32 x TCC_EA0_RDREQ_DRAM_32B (reads), 32 x
              TCC_EA0_WRREQ_WRITE_DRAM_32B (writes); FETCH_SIZE / WRITE_SIZE
              are the L2's requests beyond itself (Infinity Cache or DRAM)

Kernel names are shortened to the function name (k_gemm_proj, ...).
"""
import csv
import glob
import os
import re
import statistics
import sys
from collections import defaultdict

SIMDS = 1024          # 256 CUs x 4 SIMDs (MI355X)
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
        if "SQ_VALU_MFMA_BUSY_CYCLES" in c and c.get("GRBM_GUI_ACTIVE"):
            derived.append(("MFMA busy", f"{100 * c['SQ_VALU_MFMA_BUSY_CYCLES'] / (SIMDS * c['GRBM_GUI_ACTIVE']):.1f}% of SIMD cycles"))
        if "SQ_ACTIVE_INST_VALU" in c and c.get("SQ_BUSY_CU_CYCLES"):
            derived.append(("VALU busy", f"{100 * c['SQ_ACTIVE_INST_VALU'] / (4 * c['SQ_BUSY_CU_CYCLES']):.1f}%"))
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


if __name__ == "__main__":
    if len(sys.argv) >= 3 and sys.argv[1] == "trace":
        trace(sys.argv[2])
    elif len(sys.argv) >= 3 and sys.argv[1] == "pmc":
        pmc(sys.argv[2:])
    else:
        print(__doc__)
        sys.exit(2)
