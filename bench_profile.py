"""Summaries of rocprofv3 output for the committed profiles.

    python bench_profile.py stats   --csv KERNEL_STATS.csv [--match SUBSTR] --command CMD --out FILE
    python bench_profile.py stats   --by-grid --csv KERNEL_TRACE.csv --command CMD --out FILE
    python bench_profile.py traffic --fetch FETCH.csv --write WRITE.csv --match SUBSTR
                                   --command CMD --out FILE
    python bench_profile.py counters --csv PASS1.csv [--csv PASS2.csv ...] --kernel LABEL=SUBSTR
                                     [--skip N] --command CMD --out FILE

``stats`` condenses a ``--kernel-trace --stats`` kernel_stats.csv to the
kernels' call counts and average durations (with ``--by-grid``, the
kernel_trace.csv of the same run, one row per kernel and grid size, so that
one kernel launched at several shapes is not averaged across them).  ``counters`` averages the
counters of one or more ``--pmc`` passes per kernel and derives the clock,
the MFMA busy fraction and the LDS bank-conflict rate.  ``traffic`` turns two
``--pmc FETCH_SIZE`` / ``--pmc WRITE_SIZE`` counter_collection.csv files into
L2-miss bytes per launch of the matched kernel (the fabric side of the L2:
the last-level cache serves part of them, HBM the rest).  Both counters report KiB per
dispatch; each is calibrated against the plain 1 GiB copy that
``bench.py --pmc-pass`` runs after the kernel (read 1 GiB, write 1 GiB), so
bytes = counter_KiB * 1024 * (2**30 / copy_counter_bytes).  The summary
records the hash of the kernel's sources; bench.py reports the traffic only
while that hash still matches.
"""

import argparse
import re
import csv
import os
import statistics
import sys
import time

COPY_BYTES = 1 << 30
COPY_MATCH = "copyBuffer"


def _rows(path):
    with open(path, newline="") as fh:
        return list(csv.DictReader(fh))


_OUT_TYPES = {"f": "float", "DF16_": "_Float16", "DF16b": "__bf16"}


def short_name(name):
    """A kernel name without namespaces and parameter lists.

    The profiler demangles most names; ones whose template arguments include
    _Float16 or __bf16 stay mangled, and the product kernels among them are
    spelled out here from their template arguments.
    """
    m = re.match(r"_ZN6fp16mc12_GLOBAL__N_114gemm_nt_kernelINS0_3CfgI((?:Li\d+E)+)EENS0_\d+(In\w+?)E"
                 r"(f|DF16_|DF16b)((?:Lb[01]E)+)", name)
    if m:
        cfg = ", ".join(re.findall(r"Li(\d+)E", m.group(1)))
        flags = ", ".join("true" if b == "1" else "false" for b in re.findall(r"Lb([01])E", m.group(4)))
        return f"gemm_nt_kernel<Cfg<{cfg}>, {m.group(2)}, {_OUT_TYPES[m.group(3)]}, {flags}>"
    m = re.match(r"_ZN12_GLOBAL__N_19mfma_loopILi(\d+)EE", name)
    if m:
        return f"mfma_loop<{m.group(1)}> (bench_ceiling.hip)"
    n = name.replace("void ", "", 1).replace("fp16mc::(anonymous namespace)::", "")
    n = n.replace("(anonymous namespace)::", "")
    depth = 0
    for i, ch in enumerate(n):          # drop the parameter list after the template arguments
        if ch == "<":
            depth += 1
        elif ch == ">":
            depth -= 1
        elif ch == "(" and depth == 0 and i > 0:
            return n[:i]
    return n


def kernel_stats(path, match=None):
    out = []
    for r in _rows(path):
        if match and match not in r["Name"]:
            continue
        out.append({"name": r["Name"], "calls": int(r["Calls"]), "avg_ns": float(r["AverageNs"]),
                    "min_ns": float(r["MinNs"]), "max_ns": float(r["MaxNs"])})
    return out


def kernel_stats_by_grid(path, match=None):
    """The same figures from a kernel_trace.csv, one row per kernel and grid size
    (launches of one kernel at different shapes stay apart)."""
    groups = {}
    for r in _rows(path):
        if match and match not in r["Kernel_Name"]:
            continue
        wgs = int(r["Grid_Size_X"]) * int(r["Grid_Size_Y"]) * int(r["Grid_Size_Z"]) // max(
            1, int(r["Workgroup_Size_X"]) * int(r["Workgroup_Size_Y"]) * int(r["Workgroup_Size_Z"]))
        ns = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
        groups.setdefault((r["Kernel_Name"], wgs), []).append(ns)
    return [{"name": name, "workgroups": wgs, "calls": len(v), "avg_ns": sum(v) / len(v),
             "min_ns": float(min(v)), "max_ns": float(max(v))} for (name, wgs), v in groups.items()]


def counter_per_dispatch(path, match):
    vals = {}
    for r in _rows(path):
        if match in r["Kernel_Name"]:
            key = r["Dispatch_Id"]
            vals[key] = vals.get(key, 0.0) + float(r["Counter_Value"])
    return list(vals.values())


def traffic(fetch_csv, write_csv, match):
    f_k = counter_per_dispatch(fetch_csv, match)
    w_k = counter_per_dispatch(write_csv, match)
    f_c = counter_per_dispatch(fetch_csv, COPY_MATCH)
    w_c = counter_per_dispatch(write_csv, COPY_MATCH)
    if not (f_k and w_k and f_c and w_c):
        raise SystemExit("counter files lack the kernel or the calibration copy")
    f_scale = COPY_BYTES / (statistics.mean(f_c) * 1024)
    w_scale = COPY_BYTES / (statistics.mean(w_c) * 1024)
    fetch_b = statistics.mean(f_k) * 1024 * f_scale
    write_b = statistics.mean(w_k) * 1024 * w_scale
    return {"fetch_kib_raw": statistics.mean(f_k), "write_kib_raw": statistics.mean(w_k),
            "fetch_scale": f_scale, "write_scale": w_scale, "fetch_bytes": fetch_b, "write_bytes": write_b,
            "l2_miss_bytes_per_launch": fetch_b + write_b, "dispatches": (len(f_k), len(w_k))}


N_SIMDS = 1024            # 256 CUs x 4 SIMDs


def counter_dispatches(paths, match, skip):
    """{dispatch id: {counter: value, '_dur_ns': duration}} for the matched kernel, from
    one or more counter_collection.csv files (one per pass), first ``skip`` dispatches
    of each file dropped (clock ramp)."""
    merged = []
    for path in paths:
        per = {}
        for r in _rows(path):
            if match not in r["Kernel_Name"]:
                continue
            d = per.setdefault(int(r["Dispatch_Id"]), {})
            d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
            d["_dur_ns"] = float(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
        ids = sorted(per)[skip:]
        merged.append([per[i] for i in ids])
    return merged


def counters(paths, match, skip, trace_us=None):
    """Mean of every counter over the kept dispatches of each pass, plus derived figures:
    clock (busy MFMA cycles / MfmaUtil gives the GRBM_GUI_ACTIVE of one XCD, divided by the
    dispatch's duration), MFMA busy %, LDS bank-conflict cycles per LDS-active cycle."""
    out, derived = {}, {}
    durs = []
    for passes in counter_dispatches(paths, match, skip):
        if not passes:
            raise SystemExit(f"no dispatch of {match!r} left after skipping {skip}")
        keys = sorted({k for d in passes for k in d if k != "_dur_ns"})
        for k in keys:
            out[k] = statistics.mean(d[k] for d in passes if k in d)
        durs += [d["_dur_ns"] for d in passes]
        if "MfmaUtil" in keys and "SQ_VALU_MFMA_BUSY_CYCLES" in keys:
            clocks = [d["SQ_VALU_MFMA_BUSY_CYCLES"] / (N_SIMDS * d["MfmaUtil"] / 100.0) / d["_dur_ns"]
                      for d in passes if d.get("MfmaUtil", 0) > 0]
            if clocks:
                derived["clock_ghz_under_counters"] = statistics.mean(clocks)
            cycles = [d["SQ_VALU_MFMA_BUSY_CYCLES"] / (N_SIMDS * d["MfmaUtil"] / 100.0)
                      for d in passes if d.get("MfmaUtil", 0) > 0]
            if cycles:
                derived["active_cycles_per_xcd"] = statistics.mean(cycles)
                if trace_us:
                    derived["clock_ghz_at_trace_duration"] = statistics.mean(cycles) / (trace_us * 1e3)
    derived["dispatches_used_per_pass"] = len(durs) // max(1, len(paths))
    derived["duration_us_under_counters"] = statistics.mean(durs) / 1e3
    if "MfmaUtil" in out:
        derived["mfma_busy_pct"] = out["MfmaUtil"]
    if "SQ_LDS_BANK_CONFLICT" in out and "SQ_LDS_IDX_ACTIVE" in out and out["SQ_LDS_IDX_ACTIVE"] > 0:
        derived["lds_conflict_cycles_per_active_cycle"] = out["SQ_LDS_BANK_CONFLICT"] / out["SQ_LDS_IDX_ACTIVE"]
    return out, derived


def main(argv=None):
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("stats")
    s.add_argument("--csv", required=True, help="kernel_stats.csv, or kernel_trace.csv with --by-grid")
    s.add_argument("--by-grid", action="store_true", help="--csv is a kernel_trace.csv: one row per grid size")
    s.add_argument("--match", default=None)
    s.add_argument("--command", required=True)
    s.add_argument("--out", required=True)
    t = sub.add_parser("traffic")
    t.add_argument("--fetch", required=True)
    t.add_argument("--write", required=True)
    t.add_argument("--match", required=True)
    t.add_argument("--algorithmic-bytes", type=float, required=True)
    t.add_argument("--expected-fetch-bytes", type=float, default=None,
                   help="the fetch the tiling cannot avoid (reported beside the measured one)")
    t.add_argument("--expected-note", default="", help="how --expected-fetch-bytes follows from the tiling")
    t.add_argument("--source-hash", required=True)
    t.add_argument("--command", required=True)
    t.add_argument("--out", required=True)
    c = sub.add_parser("counters")
    c.add_argument("--csv", action="append", required=True, help="counter_collection.csv, one per pass")
    c.add_argument("--kernel", action="append", required=True,
                   help="LABEL[:SKIP]=SUBSTRING of the kernel name (SKIP overrides --skip)")
    c.add_argument("--skip", type=int, default=0, help="dispatches of each kernel dropped per pass")
    c.add_argument("--trace-csv", default=None,
                   help="kernel_trace.csv of an uncounted run of the same program: the mean duration of "
                        "the kept dispatches gives the clock")
    c.add_argument("--source-hash", default="")
    c.add_argument("--command", required=True)
    c.add_argument("--out", required=True)
    a = ap.parse_args(argv)
    stamp = time.strftime("%Y-%m-%d")
    if a.cmd == "stats":
        ks = kernel_stats_by_grid(a.csv, a.match) if a.by_grid else kernel_stats(a.csv, a.match)
        lines = [f"# rocprofv3 kernel statistics ({stamp})", f"# command: {a.command}",
                 "# gemm_nt_kernel<tile configuration, operand type, output type, accumulate,"
                 " A stored K x M, B stored K x N>", ""]
        if a.by_grid:
            lines += ["| kernel | workgroups | calls | avg us | min us | max us |", "|---|---|---|---|---|---|"]
        else:
            lines += ["| kernel | calls | avg us | min us | max us |", "|---|---|---|---|---|"]
        for k in sorted(ks, key=lambda k: -k["avg_ns"] * k["calls"]):
            grid = f" {k['workgroups']} |" if a.by_grid else ""
            lines.append(f"| `{short_name(k['name'])[:160]}` |{grid} {k['calls']} | {k['avg_ns'] / 1e3:.2f} | "
                         f"{k['min_ns'] / 1e3:.2f} | {k['max_ns'] / 1e3:.2f} |")
        text = "\n".join(lines) + "\n"
    elif a.cmd == "counters":
        lines = [f"# rocprofv3 counters per dispatch ({stamp}), mean over the kept dispatches",
                 f"# command (one pass per --pmc set): {a.command}",
                 "# the first dispatches of each kernel in each pass are dropped (clock ramp)",
                 "# active_cycles_per_xcd = SQ_VALU_MFMA_BUSY_CYCLES / (1024 SIMDs x MfmaUtil/100), i.e. the",
                 "#   GRBM_GUI_ACTIVE of one XCD; clock = those cycles over a duration: the dispatch's own under",
                 "#   counter collection (which stretches it), or the average of an uncounted kernel trace;",
                 "# mfma_busy_pct = MfmaUtil = busy MFMA cycles / (GRBM_GUI_ACTIVE x 1024 SIMDs)"]
        if a.source_hash:
            lines.append(f"source_hash = {a.source_hash}")
        for spec in a.kernel:
            label, match = spec.split("=", 1)
            skip = a.skip
            if ":" in label:
                label, skip = label.split(":", 1)
                skip = int(skip)
            lines.append(f"[{label}]  match: {match}; first {skip} dispatches per pass dropped")
            trace_us = None
            if a.trace_csv:
                durs = [int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
                        for r in _rows(a.trace_csv) if match in r["Kernel_Name"]][skip:]
                if durs:
                    trace_us = statistics.mean(durs) / 1e3
                    lines.append(f"{label}.trace_avg_us = {trace_us:.2f}  (uncounted run, same dispatches kept)")
            raw, der = counters(a.csv, match, skip, trace_us)
            for k, v in der.items():
                lines.append(f"{label}.{k} = {v:.4g}" if isinstance(v, float) else f"{label}.{k} = {v}")
            for k, v in raw.items():
                lines.append(f"{label}.raw.{k} = {v:.6g}")
        text = "\n".join(lines) + "\n"
    else:
        tr = traffic(a.fetch, a.write, a.match)
        text = "\n".join([
            f"# L2-miss traffic per launch from rocprofv3 --pmc FETCH_SIZE and --pmc WRITE_SIZE ({stamp})",
            "# (bytes the L2 requests from and writes to the fabric; the 256 MB last-level cache serves",
            "#  part of the reads, so HBM itself moves at most this much)",
            f"# command (one pass per counter): {a.command}",
            f"# kernel match: {a.match}",
            "# calibration: a 1 GiB device copy (read 1 GiB, write 1 GiB) in the same run",
            f"fetch_kib_raw = {tr['fetch_kib_raw']:.1f}",
            f"write_kib_raw = {tr['write_kib_raw']:.1f}",
            f"fetch_scale = {tr['fetch_scale']:.4f}",
            f"write_scale = {tr['write_scale']:.4f}",
            f"fetch_bytes = {tr['fetch_bytes']:.0f}",
            f"write_bytes = {tr['write_bytes']:.0f}",
            f"l2_miss_bytes_per_launch = {tr['l2_miss_bytes_per_launch']:.0f}",
            f"algorithmic_bytes_per_launch = {a.algorithmic_bytes:.0f}",
            f"traffic_over_algorithmic = {tr['l2_miss_bytes_per_launch'] / a.algorithmic_bytes:.3f}",
            *([f"# expected fetch: {a.expected_note}",
               f"expected_fetch_bytes = {a.expected_fetch_bytes:.0f}",
               f"fetch_over_expected = {tr['fetch_bytes'] / a.expected_fetch_bytes:.4f}"]
              if a.expected_fetch_bytes else []),
            f"dispatches = {tr['dispatches'][0]} fetch, {tr['dispatches'][1]} write",
            f"source_hash = {a.source_hash}",
        ]) + "\n"
    os.makedirs(os.path.dirname(os.path.abspath(a.out)), exist_ok=True)
    with open(a.out, "w") as fh:
        fh.write(text)
    sys.stdout.write(text)


if __name__ == "__main__":
    main()
