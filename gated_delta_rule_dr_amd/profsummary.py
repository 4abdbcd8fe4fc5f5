"""Summarise rocprofv3 output of ``bench.py`` runs into the short text records kept under
``profiles/``.

    python -m gated_delta_rule_dr_amd.profsummary trace  <kernel_stats.csv> <out.md> "<command>"
    python -m gated_delta_rule_dr_amd.profsummary traffic <fetch_counter_collection.csv> \\
        <write_counter_collection.csv> <copy_ref_mib> <kernel-substring>[;<kernel-substring>...] \\
        <source-files;...> <algorithmic-bytes-per-call> <out.json> "<fetch command>" "<write command>"
    python -m gated_delta_rule_dr_amd.profsummary mfma <counter_collection.csv> <kernel_stats.csv> \\
        <kernel-substring>[;...] <out.md> "<counter command>" "<trace command>"

    python -m gated_delta_rule_dr_amd.profsummary l2path <out.md> <kernel-substring>[;...] \
        "<command 1>" <counter_collection 1.csv> ["<command 2>" <counter_collection 2.csv> ...]

``l2path`` tabulates the vector-memory counters of one dispatch per kernel (averaged over the
dispatches profiled, summed over the device) from any number of counter runs, and derives the
average L1-miss latency TCP_TCC_READ_REQ_LATENCY_sum / TCP_TCC_READ_REQ_sum (cycles), the L2 hit
rate TCC_HIT_sum / (TCC_HIT_sum + TCC_MISS_sum) and the fraction of CU cycles the L1 stalled on
pending L2 data, TCP_PENDING_STALL_CYCLES_sum / (GRBM_GUI_ACTIVE / 8 XCDs x 256 CUs).

``mfma`` reports, per kernel, the matrix-core counters of one dispatch (averaged over the
dispatches profiled): SQ_INSTS_VALU_MFMA_MOPS_F16 (units of 512 flops), SQ_INSTS_MFMA,
SQ_VALU_MFMA_BUSY_CYCLES, SQ_BUSY_CYCLES and GRBM_GUI_ACTIVE, with the counted fp16 matrix
flops divided by the kernel's average duration from a kernel trace of the same command, against
the 2.5 PFLOP/s dense fp16 peak.

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
    for pattern in patterns.split(";"):
        f_kib, nf = _kernel_avg(fr, "FETCH_SIZE", pattern)
        w_kib, nw = _kernel_avg(wr, "WRITE_SIZE", pattern)
        kernels[pattern] = {"fetch_size_kib_per_dispatch": f_kib, "write_size_kib_per_dispatch": w_kib,
                            "dispatches": [nf, nw], "hbm_read_bytes": f_kib * 1024.0 * f_fac,
                            "hbm_write_bytes": w_kib * 1024.0 * w_fac}
        read_b += f_kib * 1024.0 * f_fac
        write_b += w_kib * 1024.0 * w_fac
    # the kernel sources the record covers (';'-separated), hashed in order as bench.source_hash does
    h = hashlib.sha256()
    for path in source.split(";"):
        with open(path, "rb") as f:
            h.update(f.read())
    sha = h.hexdigest()[:16]
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


MFMA_COUNTERS = ("SQ_INSTS_VALU_MFMA_MOPS_F16", "SQ_INSTS_MFMA", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_BUSY_CYCLES",
                 "GRBM_GUI_ACTIVE")


def mfma(counter_csv, stats_csv, patterns, out_md, cmd_counters, cmd_trace):
    rows = _rows(counter_csv)
    stats = _rows(stats_csv)
    lines = [
        "# Matrix-core counters per dispatch",
        "",
        f"Counters: `{cmd_counters}`",
        "",
        f"Durations: `{cmd_trace}`",
        "",
        "Counted fp16 matrix flops = SQ_INSTS_VALU_MFMA_MOPS_F16 x 512; rate = flops / average duration;",
        "peak 2.5 PFLOP/s (dense fp16).",
        "",
        "| kernel | " + " | ".join(MFMA_COUNTERS) + " | avg duration (us) | counted TFLOP/s | fraction of peak |",
        "|---|" + "---|" * (len(MFMA_COUNTERS) + 3),
    ]
    for pattern in patterns.split(";"):
        vals = []
        for c in MFMA_COUNTERS:
            v, _ = _kernel_avg(rows, c, pattern)
            vals.append(v)
        durs = [float(r["AverageNs"]) for r in stats if pattern in r["Name"]]
        dur_ns = durs[0] if durs else float("nan")
        flops = vals[0] * 512.0
        tf = flops / dur_ns / 1e3 if durs else float("nan")
        lines.append(f"| `{pattern}` | " + " | ".join(f"{v:.4g}" for v in vals) +
                     f" | {dur_ns / 1e3:.1f} | {tf:.1f} | {tf / 2500.0:.4f} |")
    with open(out_md, "w") as f:
        f.write("\n".join(lines) + "\n")


def l2path(out_md, patterns, *runs):
    pats = patterns.split(";")
    cmds, vals = [], {p: {} for p in pats}
    for cmd, path in zip(runs[0::2], runs[1::2]):
        cmds.append(cmd)
        rows = _rows(path)
        for p in pats:
            for c in sorted({r["Counter_Name"] for r in rows if p in r["Kernel_Name"]}):
                vals[p][c] = _kernel_avg(rows, c, p)[0]
    counters = sorted({c for d in vals.values() for c in d})
    lines = ["# Vector-memory path counters per dispatch", ""]
    lines += [f"Run {i + 1}: `{c}`" for i, c in enumerate(cmds)]
    lines += ["", "| kernel | " + " | ".join(counters) + " | L1-miss latency (cycles) | L2 hit rate | L1 pending-stall fraction |",
              "|---|" + "---|" * (len(counters) + 3)]
    for p in pats:
        d = vals[p]
        lat = d["TCP_TCC_READ_REQ_LATENCY_sum"] / d["TCP_TCC_READ_REQ_sum"] if "TCP_TCC_READ_REQ_sum" in d else float("nan")
        hit = d["TCC_HIT_sum"] / (d["TCC_HIT_sum"] + d["TCC_MISS_sum"]) if "TCC_HIT_sum" in d else float("nan")
        stall = (d["TCP_PENDING_STALL_CYCLES_sum"] / (d["GRBM_GUI_ACTIVE"] / 8 * 256)
                 if "TCP_PENDING_STALL_CYCLES_sum" in d and "GRBM_GUI_ACTIVE" in d else float("nan"))
        lines.append(f"| `{p}` | " + " | ".join(f"{d.get(c, float('nan')):.4g}" for c in counters) +
                     f" | {lat:.0f} | {hit:.3f} | {stall:.3f} |")
    with open(out_md, "w") as f:
        f.write("\n".join(lines) + "\n")


if __name__ == "__main__":
    mode = sys.argv[1]
    if mode == "trace":
        trace(*sys.argv[2:5])
    elif mode == "traffic":
        traffic(*sys.argv[2:12])
    elif mode == "mfma":
        mfma(*sys.argv[2:8])
    elif mode == "l2path":
        l2path(*sys.argv[2:])
    else:
        raise SystemExit(__doc__)
