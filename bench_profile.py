"""Summaries of rocprofv3 output for the committed profiles.

    python bench_profile.py stats   --csv KERNEL_STATS.csv --match SUBSTR --command CMD --out FILE
    python bench_profile.py traffic --fetch FETCH.csv --write WRITE.csv --match SUBSTR
                                                     --command CMD --out FILE

``stats`` condenses a ``--kernel-trace --stats`` kernel_stats.csv to the
kernels' call counts and average durations.  ``traffic`` turns two
``--pmc FETCH_SIZE`` / ``--pmc WRITE_SIZE`` counter_collection.csv files into
HBM bytes per launch of the matched kernel.  Both counters report KiB per
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
    n = name.replace("void ", "", 1).replace("fp16mc::(anonymous namespace)::", "")
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
            "hbm_bytes_per_launch": fetch_b + write_b, "dispatches": (len(f_k), len(w_k))}


def main(argv=None):
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("stats")
    s.add_argument("--csv", required=True)
    s.add_argument("--match", default=None)
    s.add_argument("--command", required=True)
    s.add_argument("--out", required=True)
    t = sub.add_parser("traffic")
    t.add_argument("--fetch", required=True)
    t.add_argument("--write", required=True)
    t.add_argument("--match", required=True)
    t.add_argument("--algorithmic-bytes", type=float, required=True)
    t.add_argument("--source-hash", required=True)
    t.add_argument("--command", required=True)
    t.add_argument("--out", required=True)
    a = ap.parse_args(argv)
    stamp = time.strftime("%Y-%m-%d")
    if a.cmd == "stats":
        ks = kernel_stats(a.csv, a.match)
        lines = [f"# rocprofv3 kernel statistics ({stamp})", f"# command: {a.command}",
                 "# gemm_nt_kernel<tile configuration, operand type, output type, accumulate,"
                 " A stored K x M, B stored K x N>", "",
                 "| kernel | calls | avg us | min us | max us |", "|---|---|---|---|---|"]
        for k in sorted(ks, key=lambda k: -k["avg_ns"] * k["calls"]):
            lines.append(f"| `{short_name(k['name'])[:160]}` | {k['calls']} | {k['avg_ns'] / 1e3:.2f} | "
                         f"{k['min_ns'] / 1e3:.2f} | {k['max_ns'] / 1e3:.2f} |")
        text = "\n".join(lines) + "\n"
    else:
        tr = traffic(a.fetch, a.write, a.match)
        text = "\n".join([
            f"# HBM traffic per launch from rocprofv3 --pmc FETCH_SIZE and --pmc WRITE_SIZE ({stamp})",
            f"# command (one pass per counter): {a.command}",
            f"# kernel match: {a.match}",
            "# calibration: a 1 GiB device copy (read 1 GiB, write 1 GiB) in the same run",
            f"fetch_kib_raw = {tr['fetch_kib_raw']:.1f}",
            f"write_kib_raw = {tr['write_kib_raw']:.1f}",
            f"fetch_scale = {tr['fetch_scale']:.4f}",
            f"write_scale = {tr['write_scale']:.4f}",
            f"fetch_bytes = {tr['fetch_bytes']:.0f}",
            f"write_bytes = {tr['write_bytes']:.0f}",
            f"hbm_bytes_per_launch = {tr['hbm_bytes_per_launch']:.0f}",
            f"algorithmic_bytes_per_launch = {a.algorithmic_bytes:.0f}",
            f"traffic_over_algorithmic = {tr['hbm_bytes_per_launch'] / a.algorithmic_bytes:.3f}",
            f"dispatches = {tr['dispatches'][0]} fetch, {tr['dispatches'][1]} write",
            f"source_hash = {a.source_hash}",
        ]) + "\n"
    os.makedirs(os.path.dirname(os.path.abspath(a.out)), exist_ok=True)
    with open(a.out, "w") as fh:
        fh.write(text)
    sys.stdout.write(text)


if __name__ == "__main__":
    main()
