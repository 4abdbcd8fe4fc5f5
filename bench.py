#!/usr/bin/env python3
"""Benchmark of the gated delta-rule hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--no-decode] [--all]

One step is one chunked forward (dr_chunk_fwd) over the scalar-gate Gated DeltaNet prefill
batch B=4, H=16, T=4096, dk=dv=128, bf16 q/k/v, fp32 gates and state, chunk 64.  W untimed
warm-up steps run first; K steps are then timed between two device synchronisations with HIP
events on the stream the kernels are launched on.  Two independently drawn input sets
alternate so that the 194 MiB batch is not served from the 256 MB last-level cache.

The single JSON line printed at the end carries:
  value        prefill tokens/s (B*H*T per second of kernel time)
  roofline     one forward call (its two kernels: the chunk-parallel prep and the chunk scan)
               against HBM bandwidth: algorithmic bytes per call (compulsory input/output
               bytes) / average call duration, peak 8 TB/s, plus the counter-measured HBM
               traffic of both kernels when a counter summary for the current kernel source is
               committed under profiles/
  mfma         algorithmic matrix flops / time against the 2.5 PFLOP/s dense fp16/bf16 peak
  decode       1000 single-token steps for 256 sequences x 32 heads (steps/s, GB/s, fraction
               of HBM peak)
  cpu_baseline the fp64 oracle on a bounded sample of the same workload, one thread
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_PEAK_TFLOPS = 2500.0  # dense fp16 / bf16
METRIC = "prefill tokens/s (B·H·T/s) + MFMA % peak; decode steps/s + HBM GB/s % peak"
PREFILL = "gdn_scalar_bf16_t4k"
DECODE = "decode_kda_n256_h32"
CHUNK_SRC = os.path.join(ROOT, "gated_delta_rule_dr_amd", "csrc", "chunk.hip")
DECODE_SRC = os.path.join(ROOT, "gated_delta_rule_dr_amd", "csrc", "decode.hip")
PROFILES = os.path.join(ROOT, "profiles")


def n_states(wl) -> int:
    """States of one forward: one per batch row, or one per sequence of a packed workload."""
    if wl.seq_median > 0:
        from gated_delta_rule_dr_amd.workloads import seq_lengths

        return len(seq_lengths(wl))
    return wl.B


def algorithmic_bytes(wl) -> int:
    """Compulsory HBM bytes of one forward: q, k, v in their storage type, every gate once, the
    fp32 output, S0 when given and S_T (one state per batch row or packed sequence)."""
    th = wl.B * wl.T * wl.H
    qkv = 2 if wl.qkv_dtype == "bf16" else 4
    per_tok = qkv * (2 * wl.dk + wl.dv) + 4 * wl.dv
    per_tok += 4 * (wl.dk if wl.decay_channel else 1)
    per_tok += 4 * (wl.dk if wl.erase_channel else 1)
    per_tok += 4 * wl.dv if wl.write == "channel" else 0
    state = n_states(wl) * wl.H * wl.dk * wl.dv * 4
    return th * per_tok + state * (2 if wl.s0_std > 0 else 1)


def algorithmic_flops(wl) -> float:
    """Matrix flops of the chunk form per chunk of C = 64 (fixed for counting):
    symmetric gates 10 C^2 d + 6 C d^2 + C^3 / 3, separate erase/write 16 C^2 d + 8 C d^2 + C^3 / 3."""
    C, d = 64, wl.dk
    general = (wl.erase_channel and not wl.rate_sqrt) or wl.write == "channel"
    per_chunk = (16 * C * C * d + 8 * C * d * d) if general else (10 * C * C * d + 6 * C * d * d)
    per_chunk += C ** 3 / 3
    return wl.B * wl.H * (wl.T / C) * per_chunk


def gate_desc(wl) -> str:
    decay = "per channel" if wl.decay_channel else "per head"
    if wl.rate_sqrt:
        return f"fp32 decay {decay}, FG2 per-channel rate (sqrt into k and v)"
    if wl.write == "channel":
        return f"fp32 decay {decay}, erase {'per channel' if wl.erase_channel else 'per head'}, write per channel"
    return f"fp32 decay {decay}, one per-head erase/write gate" if wl.decay_channel else "fp32 per head"


def backward_bytes(wl) -> int:
    """Compulsory HBM bytes of one gradient call: the forward's inputs, dO (fp32), and the fp32
    gradients of q, k, v and every gate (S0 / dS_T / dS0 when the forward has an S0)."""
    th = wl.B * wl.T * wl.H
    qkv = 2 if wl.qkv_dtype == "bf16" else 4
    gates = 4 * ((wl.dk if wl.decay_channel else 1) + (wl.dk if wl.erase_channel else 1)
                 + (wl.dv if wl.write == "channel" else 0))
    per_tok = qkv * (2 * wl.dk + wl.dv) + 4 * wl.dv + 4 * (2 * wl.dk + wl.dv) + 2 * gates
    state = wl.B * wl.H * wl.dk * wl.dv * 4
    return th * per_tok + (3 * state if wl.s0_std > 0 else state)


def time_backward(dr, torch, wl, steps, warmup):
    from gated_delta_rule_dr_amd.workloads import generate

    x = generate(wl, device="cuda")
    g = torch.Generator(device="cuda").manual_seed(wl.seed + 77)
    dO = torch.randn((wl.B, wl.T, wl.H, wl.dv), generator=g, device="cuda")
    dST = torch.randn((wl.B, wl.H, wl.dk, wl.dv), generator=g, device="cuda")
    call = lambda: dr.chunk_bwd(x["q"], x["k"], x["v"], x["log_decay"], x["erase"], x["write"], x["S0"],
                                dO=dO, dS_T=dST)
    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        call()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / 1e3 / steps


def cpu_baseline_backward(wl, tokens):
    """The fp64 adjoint oracle on the first `tokens` tokens of every (b, h) of the workload."""
    from threadpoolctl import threadpool_limits

    from gated_delta_rule_dr_amd.workloads import generate
    from oracle import recurrence_bwd

    sample = wl.replace(T=tokens)
    inp = generate(sample)
    dO = _dO_sample(sample)
    with threadpool_limits(1):
        t0 = time.perf_counter()
        recurrence_bwd(inp["q"], inp["k"], inp["v"], inp["log_decay"], inp["erase"], inp["write"], inp["S0"], dO=dO)
        sec = time.perf_counter() - t0
    return dict(value=sample.token_heads / sec, unit="tokens/s", cores=1, kind="oracle",
                sample=f"{sample.B}x{sample.H} heads x first {tokens} tokens of {wl.name} "
                       f"({sample.token_heads} token-heads, {sec:.1f} s, fp64 numpy, 1 thread)")


def _dO_sample(wl):
    import numpy as np

    return np.random.default_rng(wl.seed + 77).standard_normal((wl.B, wl.T, wl.H, wl.dv))


def decode_bytes(wl) -> int:
    """Per decode step: the fp32 state read and written once, q/k/v, gates and the output."""
    n = wl.B * wl.H
    state = n * wl.dk * wl.dv * 4 * 2
    io = n * (2 * (2 * wl.dk + wl.dv) + 4 * wl.dv)
    io += n * 4 * (wl.dk if wl.decay_channel else 1)
    io += n * 4 * (wl.dk if wl.erase_channel else 1)
    io += n * 4 * wl.dv if wl.write == "channel" else 0
    return state + io


def source_hash(path) -> str:
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def counter_traffic(kernel: str, workload: str, src: str):
    """HBM bytes per launch from a committed counter summary, if it was taken on the current
    kernel source; otherwise None."""
    path = os.path.join(PROFILES, f"{kernel}_{workload}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_sha256_16") != source_hash(src):
        return None
    return rec.get("hbm_bytes_per_launch")


def time_prefill(dr, torch, wl, steps, warmup):
    from gated_delta_rule_dr_amd.workloads import generate

    # the second set keeps the first one's sequence lengths (they are drawn from wl.seed)
    sets = [generate(wl, device="cuda"), generate(wl, device="cuda", value_seed=wl.seed + 1000)]
    o = torch.empty((wl.B, wl.T, wl.H, wl.dv), device="cuda")
    S_T = torch.empty((n_states(wl), wl.H, wl.dk, wl.dv), device="cuda")

    def step(i):
        x = sets[i % 2]
        if "cu_seqlens" in x:
            dr.chunk_fwd_varlen(x["q"], x["k"], x["v"], x["log_decay"], x["erase"], x["write"], x["S0"],
                                cu_seqlens=x["cu_seqlens"], out=o, S_T=S_T, fg2=wl.rate_sqrt)
        else:
            dr.chunk_fwd(x["q"], x["k"], x["v"], x["log_decay"], x["erase"], x["write"], x["S0"], out=o, S_T=S_T,
                         fg2=wl.rate_sqrt)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    e0.record(stream)
    for i in range(steps):
        step(i)
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    return e0.elapsed_time(e1) / 1e3 / steps, wall


def time_decode(dr, torch, wl, steps):
    from gated_delta_rule_dr_amd.workloads import generate_decode

    inp = generate_decode(wl, steps=steps, device="cuda")
    S = inp["S0"]
    o = torch.empty((wl.B, wl.H, wl.dv), device="cuda")
    w = inp["write"]

    def step(s):
        dr.decode_step(inp["q"][s], inp["k"][s], inp["v"][s], inp["log_decay"][s], inp["erase"][s],
                       None if w is None else w[s], S=S, o=o)

    for s in range(3):  # warm-up on the first inputs; the state keeps evolving
        step(s)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for s in range(steps):
        step(s)
    e1.record(stream)
    torch.cuda.synchronize()
    sec = e0.elapsed_time(e1) / 1e3
    del inp
    return sec / steps


def cpu_baseline(wl, tokens):
    """The fp64 oracle on the first `tokens` tokens of every (b, h) of the workload."""
    from threadpoolctl import threadpool_limits

    from gated_delta_rule_dr_amd.workloads import generate
    from oracle import recurrence, recurrence_fg2, recurrence_varlen

    sample = wl.replace(T=tokens)
    inp = generate(sample)
    args = (inp["q"], inp["k"], inp["v"], inp["log_decay"], inp["erase"], inp["write"], inp["S0"])
    with threadpool_limits(1):
        t0 = time.perf_counter()
        if "cu_seqlens" in inp:  # packed: the first `tokens` tokens, cut into the recipe's lengths
            recurrence_varlen(*args, inp["cu_seqlens"])
        elif wl.rate_sqrt:
            recurrence_fg2(inp["q"], inp["k"], inp["v"], inp["log_decay"], inp["erase"], inp["S0"])
        else:
            recurrence(*args)
        sec = time.perf_counter() - t0
    return dict(value=sample.token_heads / sec, unit="tokens/s", cores=1, kind="oracle",
                sample=f"{sample.B}x{sample.H} heads x first {tokens} tokens of {wl.name} "
                       f"({sample.token_heads} token-heads, {sec:.1f} s, fp64 numpy, 1 thread)")


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--decode-steps", type=int, default=1000)
    ap.add_argument("--cpu-tokens", type=int, default=4096)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--all", action="store_true",
                    help="also time the KDA, FG2, decoupled and packed-sequence prefill workloads")
    ap.add_argument("--backward", action="store_true",
                    help="also time the gradient call (dr_chunk_bwd) on the main workload")
    ap.add_argument("--workload", default=PREFILL,
                    help="prefill workload of the main line (default: the bench workload %(default)s)")
    ap.add_argument("--copy-ref-mib", type=int, default=0,
                    help="also run one plain elementwise copy of this many MiB (a known-size "
                         "reference for HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the recurrence shards over (batch, head) pairs with no "
              "communication, so only --gpus 1 is supported", file=sys.stderr)
        sys.exit(2)

    import torch

    import gated_delta_rule_dr_amd as dr
    from gated_delta_rule_dr_amd.workloads import workload

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    dr.abi_version()

    if args.copy_ref_mib:
        n = args.copy_ref_mib * (1 << 20) // 4
        src = torch.ones(n, device="cuda")
        dst = torch.empty_like(src)
        torch.mul(src, 1.0, out=dst)  # reads and writes copy_ref_mib MiB each
        torch.cuda.synchronize()
        del src, dst

    wl = workload(args.workload)
    if wl.steps:
        print(f"{wl.name} is a decode workload; --workload takes a prefill one", file=sys.stderr)
        sys.exit(2)
    sec, wall = time_prefill(dr, torch, wl, args.steps, args.warmup)
    tok_s = wl.token_heads / sec
    nbytes = algorithmic_bytes(wl)
    flops = algorithmic_flops(wl)
    achieved = nbytes / sec / 1e9
    traffic = counter_traffic("chunk_fwd", wl.name, CHUNK_SRC)
    line = {
        "metric": METRIC,
        "value": tok_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": sec * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16 matrix operands, fp32 accumulate and state (bf16 inputs)",
        "data": "synthetic (seeded; two alternating input sets)",
        "config": {"workload": wl.name, "B": wl.B, "H": wl.H, "T": wl.T, "dk": wl.dk, "dv": wl.dv,
                   "chunk": wl.chunk, "qkv": wl.qkv_dtype, "gates": gate_desc(wl), "o": "fp32",
                   **({"sequences": n_states(wl)} if wl.seq_median else {})},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                     "kernel": ("dr_chunk_fwd_varlen = varlen_setup_kernel + chunk_prep_kernel + scan (one call)"
                                if wl.seq_median else
                                "dr_chunk_fwd = chunk_prep_kernel + chunk_scan_sym_kernel (one call)"),
                     "algorithmic_bytes_per_launch": nbytes},
        "mfma": {"achieved_tflops": flops / sec / 1e12, "peak_tflops": MFMA_PEAK_TFLOPS,
                 "frac": flops / sec / 1e12 / MFMA_PEAK_TFLOPS, "algorithmic_flops_per_launch": flops},
        "timed_wall_s": wall,
    }
    if args.all:
        extra = {}
        for name in ("kda_channel_bf16_t16k", "fg2_channel_bf16_t16k", "gdn2_decoupled_bf16_t64k",
                     "gdn_scalar_bf16_varlen_t16k"):
            w2 = workload(name)
            s2, _ = time_prefill(dr, torch, w2, max(3, args.steps // 10), 2)
            extra[name] = {"tokens_per_s": w2.token_heads / s2, "ms": s2 * 1e3,
                           "hbm_frac": algorithmic_bytes(w2) / s2 / 1e9 / HBM_PEAK_GBS,
                           "mfma_frac": algorithmic_flops(w2) / s2 / 1e12 / MFMA_PEAK_TFLOPS}
            torch.cuda.empty_cache()
        line["other_prefill"] = extra
    if args.backward:
        bsteps = max(2, args.steps // 10)
        bsec = time_backward(dr, torch, wl, bsteps, 1)
        bbytes = backward_bytes(wl)
        line["backward"] = {"workload": wl.name, "calls": bsteps, "ms": bsec * 1e3,
                            "tokens_per_s": wl.token_heads / bsec, "hbm_frac": bbytes / bsec / 1e9 / HBM_PEAK_GBS,
                            "bytes_per_call": bbytes,
                            "kernel": "dr_chunk_bwd = bwd_token_kernel + bwd_reduce_kernel (fp32 token adjoint)"}
        if not args.no_cpu:
            line["backward"]["cpu_baseline"] = cpu_baseline_backward(wl, max(64, args.cpu_tokens // 16))
        torch.cuda.empty_cache()
    if not args.no_decode:
        dwl = workload(DECODE)
        dsec = time_decode(dr, torch, dwl, args.decode_steps)
        dbytes = decode_bytes(dwl)
        line["decode"] = {"workload": DECODE, "steps": args.decode_steps, "steps_per_s": 1.0 / dsec,
                          "us_per_step": dsec * 1e6, "GB_per_s": dbytes / dsec / 1e9,
                          "hbm_frac": dbytes / dsec / 1e9 / HBM_PEAK_GBS, "bytes_per_step": dbytes,
                          "traffic": counter_traffic("decode128_kernel", DECODE, DECODE_SRC)}
        torch.cuda.empty_cache()
    if not args.no_cpu:
        line["cpu_baseline"] = cpu_baseline(wl, args.cpu_tokens)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
