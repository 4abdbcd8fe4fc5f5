"""Summarise rocprofv3 output of ``bench.py`` runs into the short text records kept under
``profiles/``.

    python -m gated_delta_rule_dr_amd.profsummary trace  <kernel_stats.csv> <out.md> "<command>"
    python -m gated_delta_rule_dr_amd.profsummary traffic <fetch_counter_collection.csv> \\
        <write_counter_collection.csv> <copy_ref_mib> <kernel-substring>[,<kernel-substring>...] \\
        <source-file> <algorithmic-bytes-per-call> <out.json> "<fetch command>" "<write command>"

``traffic`` converts the FETCH_SIZE and WRITE_SIZE counters (KiB per dispatch) of the kernels
one call launches (each named by a substring; one dispatch of each per call) into HBM bytes
per call.  Each counter is scaled by the factor that makes it read the known
size of a plain elementwise copy profiled in the same run (``bench.py --copy-ref-mib N``:
N MiB read and N MiB written), and the record carries a hash of the kernel's source so a
stale record can be recognised.
"""
from __future__ import annotations

import csv
import hashlib
import json
import sys


def _rows(path):
    with open(path) as f:
        return list(csv.DictReader(f))


def trace(stats_csv, out_md, command):
    rows = _rows(stats_csv)
    lines = [
        "# rocprofv3 kernel trace summary",
        "",
        f"Command: `{command}`",
        "",
        "| kernel | calls | average (us) | min (us) | max (us) | share of GPU time |",
        "|---|---|---|---|---|---|",
    ]
    for r in rows:
        name = r["Name"]
        if len(name) > 90:
            name = name[:87] + "..."
        lines.append(
            f"| `{name}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
            f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} | {float(r['Percentage']):.1f}% |"
        )
    with open(out_md, "w") as f:
        f.write("\n".join(lines) + "\n")


def _copy_ref(rows, counter, copy_bytes):
    cand = [r for r in rows if "MulFunctor<float>" in r["Kernel_Name"] and r["Counter_Name"] == counter]
    if not cand:
        raise SystemExit(f"no copy reference dispatch for {counter}")
    ref = max(cand, key=lambda r: int(r["Grid_Size"]))
    kib = float(ref["Counter_Value"])
    return copy_bytes / (kib * 1024.0), kib


def _kernel_avg(rows, counter, pattern):
    vals = [float(r["Counter_Value"]) for r in rows if pattern in r["Kernel_Name"] and r["Counter_Name"] == counter]
    if not vals:
        raise SystemExit(f"no dispatch of {pattern} with {counter}")
    return sum(vals) / len(vals), len(vals)


def traffic(fetch_csv, write_csv, copy_mib, patterns, source, alg_bytes, out_json, cmd_fetch, cmd_write):
    copy_bytes = int(copy_mib) * (1 << 20)
    fr, wr = _rows(fetch_csv), _rows(write_csv)
    f_fac, f_ref = _copy_ref(fr, "FETCH_SIZE", copy_bytes)
    w_fac, w_ref = _copy_ref(wr, "WRITE_SIZE", copy_bytes)
    kernels = {}
    read_b = write_b = 0.0
    for pattern in patterns.split(","):
        f_kib, nf = _kernel_avg(fr, "FETCH_SIZE", pattern)
        w_kib, nw = _kernel_avg(wr, "WRITE_SIZE", pattern)
        kernels[pattern] = {"fetch_size_kib_per_dispatch": f_kib, "write_size_kib_per_dispatch": w_kib,
                            "dispatches": [nf, nw], "hbm_read_bytes": f_kib * 1024.0 * f_fac,
                            "hbm_write_bytes": w_kib * 1024.0 * w_fac}
        read_b += f_kib * 1024.0 * f_fac
        write_b += w_kib * 1024.0 * w_fac
    with open(source, "rb") as f:
        sha = hashlib.sha256(f.read()).hexdigest()[:16]
    rec = {
        "kernels": kernels,
        "source": source,
        "source_sha256_16": sha,
        "copy_reference": {"bytes_each_way": copy_bytes, "fetch_size_kib": f_ref, "write_size_kib": w_ref,
                           "fetch_factor": f_fac, "write_factor": w_fac},
        "hbm_read_bytes_per_launch": read_b,
        "hbm_write_bytes_per_launch": write_b,
        "hbm_bytes_per_launch": read_b + write_b,
        "algorithmic_bytes_per_launch": int(alg_bytes),
        "traffic_over_algorithmic": (read_b + write_b) / int(alg_bytes),
        "commands": [cmd_fetch, cmd_write],
    }
    with open(out_json, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")


if __name__ == "__main__":
    mode = sys.argv[1]
    if mode == "trace":
        trace(*sys.argv[2:5])
    elif mode == "traffic":
        traffic(*sys.argv[2:12])
    else:
        raise SystemExit(__doc__)
