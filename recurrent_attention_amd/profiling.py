"""Summaries of rocprofv3 output for the library's kernels.

``python -m recurrent_attention_amd.profiling stats <kernel_stats.csv>``
    prints a markdown table of the library's kernels (calls, average, min,
    max duration) from a ``rocprofv3 --kernel-trace --stats`` CSV.
``python -m recurrent_attention_amd.profiling counters <counter_collection.csv> ...``
    prints the per-dispatch average of each counter for each of the
    library's kernels from ``rocprofv3 --pmc`` CSVs (one file per pass).
``python -m recurrent_attention_amd.profiling trace <kernel_trace.csv>``
    the same table per launch shape (family, kernel, grid), from the
    per-dispatch ``rocprofv3 --kernel-trace`` CSV, so that one kernel run
    by several parts of a program is told apart by its grid.
``python -m recurrent_attention_amd.profiling counters-md <counter_collection.csv> ...``
    the per-dispatch means as a markdown table per kernel family, with the
    matrix-core and LDS ratios derived from them (see ``derived``).
``python -m recurrent_attention_amd.profiling traffic --fetch F.csv --write W.csv
    --fetch-copy FC.csv --write-copy WC.csv --kernel NAME --copy-bytes N
    --out profiles/traffic_X.json --hash H``
    scales FETCH_SIZE / WRITE_SIZE (per dispatch) of one kernel family by
    what the same counters read for a plain device copy of N bytes each way
    (``bench.py --only copy``, a 1 GiB copy), giving HBM bytes per launch.
"""
from __future__ import annotations

import argparse
import csv
import json
import re
import statistics
import sys
from collections import defaultdict

# chunk_kernel<ChunkCfg<dk, dv, C, bf16, gate, state-only, waves>, elu1, reversed, store,
#              epilogue, sub-chunk path>
_CHUNK = (r"la::chunk_kernel<la::ChunkCfg<\d+, \d+, \d+, \w+, \d, {so}, \d+>, "
          r"\w+, \w+, {store}, \w+, {sub}>")
# chunk_main: every pass with outputs (the group-norm epilogue and the
# training forward that also stores its boundary states included);
# chunk_sub: the same passes with the sub-chunk path (vector gates)
FAMILIES = [
    ("chunk_main", re.compile(_CHUNK.format(so="false", store=r"\w+", sub="false"))),
    ("chunk_sub", re.compile(_CHUNK.format(so="false", store=r"\w+", sub="true"))),
    ("chunk_store", re.compile(_CHUNK.format(so="true", store="true", sub="false"))),
    ("chunk_state", re.compile(_CHUNK.format(so="true", store="false", sub="false"))),
    ("state_scan", re.compile(r"la::state_scan_kernel")),
    ("chunk_bwd", re.compile(r"la::bwd_kernel")),
    ("delta_chunk", re.compile(r"la::delta_chunk_kernel")),
    ("delta_decode", re.compile(r"la::delta_decode_kernel")),
    ("decode", re.compile(r"la::decode_kernel")),
    ("seq_order", re.compile(r"seq_order_kernel")),
    ("copy", re.compile(r"__amd_rocclr_copyBuffer")),
]


def family(name: str):
    for fam, rx in FAMILIES:
        if rx.search(name):
            return fam
    return None


def stats_table(path: str) -> str:
    rows = []
    with open(path) as f:
        for r in csv.DictReader(f):
            fam = family(r["Name"])
            if fam in (None, "copy"):
                continue
            rows.append((fam, r["Name"], int(r["Calls"]), float(r["AverageNs"]) / 1e3,
                         float(r["MinNs"]) / 1e3, float(r["MaxNs"]) / 1e3))
    out = ["| family | kernel | calls | avg us | min us | max us |",
           "|---|---|---:|---:|---:|---:|"]
    for fam, name, n, avg, mn, mx in rows:
        out.append(f"| {fam} | `{name}` | {n} | {avg:.2f} | {mn:.2f} | {mx:.2f} |")
    return "\n".join(out)


def trace_table(path: str) -> str:
    """calls / avg / median / min / max duration per (family, kernel, grid)
    from a per-dispatch kernel-trace CSV (the median is robust to the slower
    first launches of a run)."""
    acc = defaultdict(list)
    for r in csv.DictReader(open(path)):
        fam = family(r["Kernel_Name"])
        if fam in (None, "copy"):
            continue
        grid = int(r["Grid_Size_X"]) // max(int(r["Workgroup_Size_X"]), 1)
        dur = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
        acc[(fam, r["Kernel_Name"], grid, int(r["Workgroup_Size_X"]))].append(dur)
    out = ["| family | kernel | workgroups x threads | calls | avg us | median us | min us | max us |",
           "|---|---|---|---:|---:|---:|---:|---:|"]
    for (fam, name, grid, wg), d in sorted(acc.items(), key=lambda x: (x[0][0], x[0][2])):
        out.append(f"| {fam} | `{name}` | {grid} x {wg} | {len(d)} | {sum(d) / len(d):.2f} | "
                   f"{statistics.median(d):.2f} | {min(d):.2f} | {max(d):.2f} |")
    return "\n".join(out)


# MI355X: compute units, SIMDs per compute unit, bf16 flops per MFMA "MOP"
CUS, SIMDS = 256, 4
FLOPS_PER_MOP = 512


def derived(cs):
    """Ratios from the per-dispatch means of one kernel (None where a counter
    is missing): GRBM_GUI_ACTIVE is summed over the 8 XCDs, so a dispatch's
    busy cycles per XCD are GRBM / 8;
      mfma_busy_pct   = SQ_VALU_MFMA_BUSY_CYCLES / (busy cycles x CUs x SIMDs)
      bf16_flops      = 512 x SQ_INSTS_VALU_MFMA_MOPS_BF16 (matrix-core work done)
      lds_conflict_pct = SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE (cycles
                         lost to bank conflicts per cycle of LDS index work)."""
    g = cs.get("GRBM_GUI_ACTIVE")
    out = {}
    if g and "SQ_VALU_MFMA_BUSY_CYCLES" in cs:
        out["mfma_busy_pct"] = 100.0 * cs["SQ_VALU_MFMA_BUSY_CYCLES"] / (g / 8 * CUS * SIMDS)
    if "SQ_INSTS_VALU_MFMA_MOPS_BF16" in cs:
        out["bf16_flops"] = FLOPS_PER_MOP * cs["SQ_INSTS_VALU_MFMA_MOPS_BF16"]
    if cs.get("SQ_LDS_IDX_ACTIVE") and "SQ_LDS_BANK_CONFLICT" in cs:
        out["lds_conflict_pct"] = 100.0 * cs["SQ_LDS_BANK_CONFLICT"] / cs["SQ_LDS_IDX_ACTIVE"]
    return out


def counters_md(paths) -> str:
    rows = []
    for name, cs in counter_means(paths).items():
        fam = family(name)
        if fam in (None, "copy"):
            continue
        rows.append((fam, name, cs, derived(cs)))
    out = []
    for fam, name, cs, dv in sorted(rows):
        out.append(f"**{fam}** `{name}`\n")
        out.append("| counter | mean per dispatch |")
        out.append("|---|---:|")
        for k in sorted(cs):
            out.append(f"| {k} | {cs[k]:.6g} |")
        for k in sorted(dv):
            out.append(f"| *{k}* | {dv[k]:.4g} |")
        out.append("")
    return "\n".join(out)


def counter_means(paths):
    """{kernel name: {counter: mean per dispatch}} over the given CSVs."""
    acc = defaultdict(lambda: defaultdict(list))
    for path in paths:
        with open(path) as f:
            for r in csv.DictReader(f):
                name = r.get("Kernel_Name") or r.get("Kernel-Name") or ""
                cname = r.get("Counter_Name") or r.get("Counter-Name")
                val = r.get("Counter_Value") or r.get("Counter-Value")
                if cname is None or val is None:
                    continue
                disp = r.get("Dispatch_Id") or r.get("Dispatch-Id") or ""
                acc[name][cname].append((disp, float(val)))
    means = {}
    for name, cs in acc.items():
        means[name] = {}
        for cname, vals in cs.items():
            per_disp = defaultdict(float)
            for disp, v in vals:
                per_disp[disp] += v      # counters split over agents/XCDs add up
            means[name][cname] = sum(per_disp.values()) / max(len(per_disp), 1)
    return means


def traffic(fetch_csv, write_csv, fetch_copy_csv, write_copy_csv, kernel_family, copy_bytes,
            out, src_hash, note=""):
    fm = counter_means([fetch_csv])
    wm = counter_means([write_csv])
    fcm = counter_means([fetch_copy_csv])
    wcm = counter_means([write_copy_csv])

    def pick(means, fam, counter):
        vals = [cs[counter] for n, cs in means.items() if family(n) == fam and counter in cs]
        return max(vals) if vals else None

    f_kern = pick(fm, kernel_family, "FETCH_SIZE")
    w_kern = pick(wm, kernel_family, "WRITE_SIZE")
    f_copy = pick(fcm, "copy", "FETCH_SIZE")
    w_copy = pick(wcm, "copy", "WRITE_SIZE")
    if None in (f_kern, w_kern, f_copy, w_copy):
        raise SystemExit(f"missing counters: kernel {f_kern} {w_kern}, copy {f_copy} {w_copy}")
    f_scale = copy_bytes / f_copy      # bytes per counter unit, from the copy
    w_scale = copy_bytes / w_copy
    rec = {
        "kernel_family": kernel_family,
        "fetch_counter_per_launch": f_kern, "write_counter_per_launch": w_kern,
        "copy_bytes_each_way": copy_bytes,
        "copy_fetch_counter": f_copy, "copy_write_counter": w_copy,
        "fetch_bytes_per_launch": f_kern * f_scale,
        "write_bytes_per_launch": w_kern * w_scale,
        "hbm_bytes_per_launch": f_kern * f_scale + w_kern * w_scale,
        "source_sha256": src_hash,
        "note": note,
    }
    with open(out, "w") as fh:
        json.dump(rec, fh, indent=1)
    print(json.dumps(rec, indent=1))


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__,
                                 formatter_class=argparse.RawDescriptionHelpFormatter)
    sub = ap.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("stats")
    s.add_argument("csv")
    c = sub.add_parser("counters")
    c.add_argument("csv", nargs="+")
    tr = sub.add_parser("trace")
    tr.add_argument("csv")
    cm = sub.add_parser("counters-md")
    cm.add_argument("csv", nargs="+")
    t = sub.add_parser("traffic")
    t.add_argument("--fetch", required=True)
    t.add_argument("--write", required=True)
    t.add_argument("--fetch-copy", required=True, help="FETCH_SIZE run of bench.py --only copy")
    t.add_argument("--write-copy", required=True, help="WRITE_SIZE run of bench.py --only copy")
    t.add_argument("--kernel", required=True)
    t.add_argument("--copy-bytes", type=int, required=True)
    t.add_argument("--out", required=True)
    t.add_argument("--hash", required=True)
    t.add_argument("--note", default="")
    a = ap.parse_args(argv)
    if a.cmd == "stats":
        print(stats_table(a.csv))
    elif a.cmd == "trace":
        print(trace_table(a.csv))
    elif a.cmd == "counters-md":
        print(counters_md(a.csv))
    elif a.cmd == "counters":
        for name, cs in counter_means(a.csv).items():
            fam = family(name)
            if fam is None:
                continue
            print(f"{fam}: {name}")
            for k, v in sorted(cs.items()):
                print(f"    {k} = {v:.6g}")
    else:
        traffic(a.fetch, a.write, a.fetch_copy, a.write_copy, a.kernel, a.copy_bytes, a.out,
                a.hash, a.note)
    return 0


if __name__ == "__main__":
    sys.exit(main())
