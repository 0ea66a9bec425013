"""Summaries of rocprofv3 output for the committed performance records.

Usage (after the profiler runs listed in the summaries themselves)::

    python -m fp64_gemm_emulation_ozii_amd.profiling stats  <kernel_stats.csv> <out.txt> <command...>
    python -m fp64_gemm_emulation_ozii_amd.profiling traffic <fetch counter_collection.csv>
        <write counter_collection.csv> <copy bytes> <workload> <out.json> <command...>

``stats`` turns rocprofv3's ``--stats`` kernel table into a short text
table.  ``traffic`` turns two ``--pmc FETCH_SIZE`` / ``--pmc WRITE_SIZE``
runs into HBM bytes per launch of each kernel.  Both counters report
kilobytes per dispatch; a plain device copy of a known number of bytes in the
same run calibrates them (bytes moved / bytes reported), and the GEMM
kernel's source hash is stored so that a record taken on another kernel
version is not reused.
"""
from __future__ import annotations

import csv
import hashlib
import re
import json
import os
import statistics
import sys

PKG = os.path.dirname(os.path.abspath(__file__))


# sources that make up the int8 GEMM kernel (a change to any of them
# invalidates a stored counter record)
GEMM_SOURCES = ("gemm_i8.hip", "gemm_grid.h", "prod_mod.h")


def code_only(text: str) -> str:
    """C++ source without comments and with runs of whitespace collapsed, so
    that an edit to a comment does not count as a change of the kernel.
    (String literals in these sources hold no comment markers.)"""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def kernel_sha(names=GEMM_SOURCES, read=None) -> str:
    """Hash of the code (comments stripped) of the GEMM sources; `read(name)`
    returns a source's text (default: the file in csrc/)."""
    read = read or (lambda name: open(os.path.join(PKG, "csrc", name)).read())
    h = hashlib.sha256()
    for name in names:
        h.update(code_only(read(name)).encode())
    return h.hexdigest()[:16]


def short_name(kernel: str) -> str:
    """Kernel name without namespaces and parameters (template arguments kept,
    without spaces, so that instances stay apart)."""
    k = kernel.replace("(anonymous namespace)::", "").replace("void ", "")
    depth, cut = 0, len(k)
    for i, ch in enumerate(k):  # parameter list = first '(' outside template brackets
        if ch == "<":
            depth += 1
        elif ch == ">":
            depth -= 1
        elif ch == "(" and depth == 0:
            cut = i
            break
    k = k[:cut]
    base, _, targs = k.partition("<")
    base = base.split("::")[-1].strip()
    return base + (("<" + targs.replace(" ", "")) if targs else "")


def read_stats(path: str):
    rows = []
    with open(path) as fh:
        for r in csv.DictReader(fh):
            name = r.get("Name") or r.get("KernelName") or r.get("Kernel_Name")
            calls = int(float(r.get("Calls", 0)))
            total = float(r.get("TotalDurationNs", 0))
            avg = float(r.get("AverageNs", total / max(calls, 1)))
            pct = float(r.get("Percentage", 0))
            mn = float(r.get("MinNs", avg))
            mx = float(r.get("MaxNs", avg))
            rows.append((short_name(name), calls, total, avg, pct, mn, mx))
    return rows


def timed_average_us(trace_csv: str, kernel_prefix: str, timed: int) -> tuple[int, float]:
    """(dispatches, mean microseconds) of the last `timed` dispatches of the
    kernels whose name starts with kernel_prefix in a rocprofv3 kernel trace
    -- the calls a benchmark times after its warmup calls."""
    durs = []
    with open(trace_csv) as fh:
        for r in csv.DictReader(fh):
            if short_name(r["Kernel_Name"]).startswith(kernel_prefix):
                durs.append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    last = durs[-timed:]
    return len(last), (sum(last) / len(last) if last else float("nan"))


def write_stats(stats_csv: str, out_txt: str, command: str, trace_csv: str | None = None, timed: int = 0) -> None:
    rows = read_stats(stats_csv)
    with open(out_txt, "w") as fh:
        fh.write(f"# rocprofv3 kernel statistics\n# command: {command}\n")
        fh.write(f"# {'kernel':<28} {'calls':>6} {'avg_us':>10} {'min_us':>10} {'max_us':>10} {'total_%':>8}\n")
        for name, calls, total, avg, pct, mn, mx in sorted(rows, key=lambda r: -r[2]):
            fh.write(f"  {name:<28} {calls:>6} {avg / 1e3:>10.2f} {mn / 1e3:>10.2f} {mx / 1e3:>10.2f} {pct:>8.2f}\n")
        if trace_csv and timed > 0:
            n, avg = timed_average_us(trace_csv, "gemm_i8_kernel", timed)
            fh.write(f"# gemm_i8_kernel, the {n} timed calls (after the warmup calls): avg {avg:.2f} us\n")


def read_counter(path: str):
    """{kernel short name: [value per dispatch]} for a single-counter run."""
    per = {}
    with open(path) as fh:
        for r in csv.DictReader(fh):
            name = short_name(r.get("Kernel_Name") or r.get("Kernel-Name") or r.get("kernel_name") or "")
            val = float(r.get("Counter_Value") or r.get("Counter-Value") or r.get("value") or 0.0)
            disp = r.get("Dispatch_Id") or r.get("Dispatch-Id") or r.get("dispatch_id") or len(per)
            per.setdefault(name, {}).setdefault(disp, 0.0)
            per[name][disp] += val
    return {k: list(v.values()) for k, v in per.items()}


def write_traffic(fetch_csv: str, write_csv: str, copy_bytes: int, workload: str, out_json: str,
                  command: str) -> dict:
    fetch = read_counter(fetch_csv)
    write = read_counter(write_csv)
    copy_names = [k for k in fetch if "copy" in k.lower() or "elementwise" in k.lower()]
    if not copy_names:
        raise RuntimeError(f"no copy kernel among {sorted(fetch)}")
    copy_k = max(copy_names, key=lambda k: max(fetch[k]))
    kb = copy_bytes / 1024.0
    f_fetch = kb / max(fetch[copy_k])
    f_write = kb / max(write.get(copy_k, [kb]))
    rec = {}
    if os.path.exists(out_json):
        rec = json.load(open(out_json))
    kernels = {}
    for k in sorted(set(fetch) & set(write)):
        fb = statistics.median(fetch[k]) * 1024.0 * f_fetch
        wb = statistics.median(write[k]) * 1024.0 * f_write
        kernels[k] = {"fetch_bytes": fb, "write_bytes": wb, "hbm_bytes": fb + wb, "dispatches": len(fetch[k])}
    gemm_keys = [k for k in kernels if k.startswith("gemm_i8_kernel")]
    gemm = kernels[gemm_keys[0]] if gemm_keys else None
    rec[workload] = {
        "kernel_sha": kernel_sha(),
        "command": command,
        "copy_kernel": copy_k,
        "copy_bytes": copy_bytes,
        "fetch_scale": f_fetch,
        "write_scale": f_write,
        "gemm_hbm_bytes_per_launch": gemm["hbm_bytes"] if gemm else None,
        "kernels": kernels,
    }
    with open(out_json, "w") as fh:
        json.dump(rec, fh, indent=1, sort_keys=True)
    return rec[workload]


def write_clock(counter_csv: str, xcds: int, simds: int, timed: int, out_txt: str, command: str) -> dict:
    """Clock and MFMA occupancy of gemm_i8_kernel from one rocprofv3 --pmc run
    with GRBM_GUI_ACTIVE (summed over the XCDs), SQ_VALU_MFMA_BUSY_CYCLES and
    SQ_INSTS_MFMA: clock = GUI_ACTIVE / xcds / dispatch time; MFMA busy =
    busy cycles / (simds x GUI_ACTIVE / xcds), averaged over the last `timed`
    dispatches."""
    per = {}
    with open(counter_csv) as fh:
        for r in csv.DictReader(fh):
            if not short_name(r["Kernel_Name"]).startswith("gemm_i8_kernel"):
                continue
            d = per.setdefault(int(r["Dispatch_Id"]), {"t": (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9})
            d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    disp = [per[k] for k in sorted(per)][-timed:]
    clk, busy, mf = [], [], []
    for d in disp:
        cyc = d["GRBM_GUI_ACTIVE"] / xcds
        clk.append(cyc / d["t"])
        busy.append(d["SQ_VALU_MFMA_BUSY_CYCLES"] / (simds * cyc))
        mf.append(d["SQ_INSTS_MFMA"])
    rec = {"dispatches": len(disp), "clock_ghz": sum(clk) / len(clk) / 1e9, "mfma_busy": sum(busy) / len(busy),
           "mfma_insts": sum(mf) / len(mf), "ms": sum(d["t"] for d in disp) / len(disp) * 1e3}
    with open(out_txt, "w") as fh:
        fh.write(f"# gemm_i8_kernel clock and MFMA occupancy (rocprofv3 --pmc)\n# command: {command}\n")
        fh.write(f"# then: python -m fp64_gemm_emulation_ozii_amd.profiling clock <counter csv> {xcds} {simds} {timed} <this file>\n")
        fh.write(f"  dispatches averaged     {rec['dispatches']}\n")
        fh.write(f"  dispatch time           {rec['ms']:.3f} ms\n")
        fh.write(f"  clock (GUI_ACTIVE/{xcds}/t)  {rec['clock_ghz']:.3f} GHz\n")
        fh.write(f"  MFMA busy fraction      {rec['mfma_busy']:.3f}\n")
        fh.write(f"  MFMA instructions       {rec['mfma_insts']:.4g}\n")
    return rec


if __name__ == "__main__":
    what = sys.argv[1]
    if what == "stats":
        write_stats(sys.argv[2], sys.argv[3], " ".join(sys.argv[4:]))
    elif what == "stats-timed":  # stats csv, trace csv, timed calls, output, command
        write_stats(sys.argv[2], sys.argv[5], " ".join(sys.argv[6:]), trace_csv=sys.argv[3], timed=int(sys.argv[4]))
    elif what == "traffic":
        r = write_traffic(sys.argv[2], sys.argv[3], int(sys.argv[4]), sys.argv[5], sys.argv[6],
                          " ".join(sys.argv[7:]))
        print(json.dumps(r, indent=1))
    elif what == "clock":  # counter csv, xcds, simds, timed calls, output, command
        print(write_clock(sys.argv[2], int(sys.argv[3]), int(sys.argv[4]), int(sys.argv[5]), sys.argv[6],
                          " ".join(sys.argv[7:])))
    else:
        raise SystemExit(f"unknown mode {what}")
