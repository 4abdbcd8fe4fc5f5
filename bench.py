#!/usr/bin/env python3
"""Benchmark of the gated delta-rule hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu] [--no-decode]
                    [--no-extra] [--backward | --backward-workload NAME | --no-backward] [--segment-scan P]

One step is one chunked forward (dr_chunk_fwd) over the main prefill workload, by default the
long-context one: decoupled per-channel erase and write gates with a per-channel decay
(Gated DeltaNet-2 / FG2-GDN+), B=1, H=32, T=65536, dk=dv=128, bf16 q/k/v, fp32 gates, output and
state, chunk 64.  W untimed warm-up steps run first; K steps are then timed between two device
synchronisations with HIP events on the stream the kernels are launched on.  Two independently
drawn input sets alternate so that the batch is not served from the 256 MB last-level cache.

The single JSON line printed at the end carries:
  value         prefill tokens/s of the main workload (B*H*T per second of kernel time)
  roofline      one forward call (its two kernels: the chunk-parallel prep and the chunk scan)
                against HBM bandwidth: algorithmic bytes per call (compulsory input/output bytes)
                / average call duration, peak 8 TB/s, plus the counter-measured HBM traffic of both
                kernels when a counter summary for the current kernel source is committed under
                profiles/
  mfma          algorithmic matrix flops / time against the 2.5 PFLOP/s dense fp16/bf16 peak
  other_prefill the other prefill workloads timed the same way in the same run: scalar-gate
                Gated DeltaNet B=4 H=16 T=4096, KDA B=2 H=32 T=16384, FG2's rate at the KDA shape,
                and the packed serving prefill (16k tokens in 20 sequences)
  decode        1000 single-token steps for 256 sequences x 32 heads (steps/s, GB/s, fraction of
                HBM peak)
  backward      one gradient call (dr_chunk_bwd) on the scalar-gate workload (B=4 H=16 T=4096; or
                --backward-workload, --backward for the main one): ms per call, beside the fp32
                token-loop adjoint (chunk = 1) on the same inputs, and the fp64 adjoint oracle on a
                sample
  cpu_baseline  the fp64 oracle on the first --cpu-tokens tokens of every head of the main
                workload, the heads sharded over one worker process per host core (at most 16)
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
PREFILL = "gdn2_decoupled_bf16_t64k"
EXTRA_PREFILL = ("gdn_scalar_bf16_t4k", "kda_channel_bf16_t16k", "fg2_channel_bf16_t16k",
                 "gdn_scalar_bf16_varlen_t16k")
DECODE = "decode_kda_n256_h32"
# the chunk path's kernel sources: a counter record is used only if it was taken on these
CHUNK_SRC = [os.path.join(ROOT, "gated_delta_rule_dr_amd", "csrc", n) for n in ("chunk.hip", "scan_wide.hip")]
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


def time_backward(dr, torch, wl, steps, warmup, chunk=64):
    from gated_delta_rule_dr_amd.workloads import generate

    x = generate(wl, device="cuda")
    g = torch.Generator(device="cuda").manual_seed(wl.seed + 77)
    dO = torch.randn((wl.B, wl.T, wl.H, wl.dv), generator=g, device="cuda")
    dST = torch.randn((wl.B, wl.H, wl.dk, wl.dv), generator=g, device="cuda")
    call = lambda: dr.chunk_bwd(x["q"], x["k"], x["v"], x["log_decay"], x["erase"], x["write"], x["S0"],
                                dO=dO, dS_T=dST, chunk=chunk, fg2=wl.rate_sqrt)
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
    from oracle import recurrence_bwd, recurrence_fg2_bwd

    sample = wl.replace(T=tokens)
    inp = generate(sample)
    dO = _dO_sample(sample)
    with threadpool_limits(1):
        t0 = time.perf_counter()
        if wl.rate_sqrt:
            recurrence_fg2_bwd(inp["q"], inp["k"], inp["v"], inp["log_decay"], inp["erase"], inp["S0"], dO)
        else:
            recurrence_bwd(inp["q"], inp["k"], inp["v"], inp["log_decay"], inp["erase"], inp["write"], inp["S0"],
                           dO=dO)
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


def source_hash(paths) -> str:
    """First 16 hex digits of the sha256 of the files' bytes, concatenated in order."""
    h = hashlib.sha256()
    for path in [paths] if isinstance(paths, str) else paths:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


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


def time_segment_scan(dr, torch, wl, nseg, reps=3):
    """The segment-parallel scan composed from the library's own packed-sequence call, whose scans
    are the sliced ones (a measurement for the design record: dr_chunk_fwd runs the same algebra in
    its own full-width kernels, one workgroup per (b, h, segment) with all value columns).  Each head's T tokens split into nseg segments; because the chunk map is affine
    in (S0, v), one packed call over the first nseg - 1 segments with v = 0 and S0 = I gives the
    segments' state maps F, a second with S0 = 0 their offsets H; the segments' incoming states
    S_in[s] = F[s - 1] S_in[s - 1] + H[s - 1] are chained (nseg - 1 small matrix products per
    head, torch), and a third packed call runs all segments from their true S_in, giving o and
    S_T.  Returns (segmented ms, single-pass ms, max relative difference of o and S_T)."""
    from gated_delta_rule_dr_amd.workloads import generate

    assert wl.B == 1 and wl.dk == wl.dv and wl.T % (64 * nseg) == 0, "one sequence, whole-chunk segments"
    x = generate(wl, device="cuda")
    T, H, d = wl.T, wl.H, wl.dk
    seg = T // nseg
    cu_all = torch.arange(0, T + 1, seg, dtype=torch.int32, device="cuda")
    cu_maps = cu_all[:nseg].contiguous()
    Tm = int(cu_maps[-1])
    head = lambda t: None if t is None else t[:, :Tm].contiguous()
    qm, km, ldm, em, wm = (head(x[n]) for n in ("q", "k", "log_decay", "erase", "write"))
    vm, v0 = head(x["v"]), torch.zeros_like(head(x["v"]))
    eye = torch.eye(d, device="cuda").expand(nseg - 1, H, d, d).contiguous()
    s0 = torch.zeros((1, H, d, d), device="cuda") if x["S0"] is None else x["S0"]
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def segmented():
        _, F = dr.chunk_fwd_varlen(qm, km, v0, ldm, em, wm, eye, cu_seqlens=cu_maps, fg2=wl.rate_sqrt)
        _, Hs = dr.chunk_fwd_varlen(qm, km, vm, ldm, em, wm, None, cu_seqlens=cu_maps, fg2=wl.rate_sqrt)
        S_in = [s0[0]]
        for s in range(1, nseg):
            S_in.append(torch.matmul(F[s - 1], S_in[-1]) + Hs[s - 1])
        return dr.chunk_fwd_varlen(x["q"], x["k"], x["v"], x["log_decay"], x["erase"], x["write"],
                                   torch.stack(S_in), cu_seqlens=cu_all, fg2=wl.rate_sqrt)

    def single():
        return dr.chunk_fwd(x["q"], x["k"], x["v"], x["log_decay"], x["erase"], x["write"], x["S0"], fg2=wl.rate_sqrt)

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        best = None
        for _ in range(reps):
            e0.record()
            out = fn()
            e1.record()
            torch.cuda.synchronize()
            t = e0.elapsed_time(e1)
            best = t if best is None else min(best, t)
        return best, out

    t_seg, (o_s, S_s) = timed(segmented)
    t_one, (o_1, S_1) = timed(single)
    rel = max(float((o_s - o_1).abs().max() / o_1.abs().max()), float((S_s[-1] - S_1[0]).abs().max() / S_1.abs().max()))
    return t_seg, t_one, rel


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


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform

    return platform.processor() or "unknown"


def _oracle_shard(args):
    """Worker: the oracle on heads h0:h1 of the sample memory-mapped from `folder`; returns its
    compute interval (wall-clock start and end)."""
    folder, h0, h1, kind = args
    import numpy as np
    from threadpoolctl import threadpool_limits

    from oracle import recurrence, recurrence_fg2, recurrence_varlen

    def ld(name):
        path = os.path.join(folder, name + ".npy")
        if not os.path.exists(path):
            return None
        x = np.load(path, mmap_mode="r")
        return np.ascontiguousarray(x[:, :, h0:h1]) if name != "S0" and name != "cu_seqlens" else x

    x = {n: ld(n) for n in ("q", "k", "v", "log_decay", "erase", "write", "cu_seqlens")}
    s0 = ld("S0")
    if s0 is not None:
        s0 = np.ascontiguousarray(s0[:, h0:h1])
    with threadpool_limits(1):
        t0 = time.time()
        if kind == "varlen":
            recurrence_varlen(x["q"], x["k"], x["v"], x["log_decay"], x["erase"], x["write"], s0, x["cu_seqlens"])
        elif kind == "fg2":
            recurrence_fg2(x["q"], x["k"], x["v"], x["log_decay"], x["erase"], s0)
        else:
            recurrence(x["q"], x["k"], x["v"], x["log_decay"], x["erase"], x["write"], s0)
        t1 = time.time()
    return t0, t1


def cpu_baseline(wl, tokens, max_workers=16):
    """The fp64 oracle on the first `tokens` tokens of every (b, h) of the workload, the heads
    sharded over one worker process per host core (spawned; BLAS/OMP threads 1 each)."""
    import multiprocessing
    import shutil
    import tempfile

    import numpy as np

    from gated_delta_rule_dr_amd.workloads import generate

    sample = wl.replace(T=min(tokens, wl.T))
    inp = generate(sample)
    workers = max(1, min(len(os.sched_getaffinity(0)), max_workers, wl.H))
    folder = tempfile.mkdtemp(prefix="dr_oracle_", dir="/dev/shm" if os.path.isdir("/dev/shm") else None)
    try:
        for name, t in inp.items():
            if t is None:
                continue
            a = t.numpy() if t.dtype != __import__("torch").bfloat16 else t.float().numpy()
            np.save(os.path.join(folder, name + ".npy"), a)
        del inp
        kind = "varlen" if wl.seq_median > 0 else "fg2" if wl.rate_sqrt else "dense"
        bounds = np.linspace(0, wl.H, workers + 1).round().astype(int)
        jobs = [(folder, int(bounds[i]), int(bounds[i + 1]), kind) for i in range(workers)]
        ctx = multiprocessing.get_context("spawn")
        wall0 = time.perf_counter()
        with ctx.Pool(workers) as pool:
            spans = pool.map(_oracle_shard, jobs)
        wall = time.perf_counter() - wall0
    finally:
        shutil.rmtree(folder, ignore_errors=True)
    sec = max(e for _, e in spans) - min(s for s, _ in spans)
    return dict(value=sample.token_heads / sec, unit="tokens/s", cores=workers, kind="oracle", cpu_model=cpu_model(),
                sample=f"first {sample.T} tokens of all {wl.B}x{wl.H} heads of {wl.name} ({sample.token_heads} "
                       f"token-heads), heads sharded over {workers} worker processes: {sec:.1f} s of compute "
                       f"({wall:.1f} s with process start), fp64 numpy, 1 thread each")


def kernel_desc(wl) -> str:
    """The kernels one forward call of the workload launches."""
    general = (wl.erase_channel and not wl.rate_sqrt) or wl.write == "channel"
    prep = "chunk_prep_ch_kernel" if (wl.decay_channel or general) else "chunk_prep_scalar_kernel"
    scan = "chunk_scan_kernel" if general else "chunk_scan_sym_kernel"
    if wl.seq_median:
        return f"dr_chunk_fwd_varlen = varlen_setup_kernel + {prep} + {scan} (one call)"
    if general:  # a dense batch with separate erase and write gates: the full-width segmented scan
        return (f"dr_chunk_fwd = {prep} + chunk_scan_wide_kernel (segment maps) + wide_compose_kernel + "
                "chunk_scan_wide_kernel (segment outputs) (one call)")
    return f"dr_chunk_fwd = {prep} + {scan} (one call)"


def prefill_record(wl, sec):
    return {"tokens_per_s": wl.token_heads / sec, "ms": sec * 1e3,
            "hbm_frac": algorithmic_bytes(wl) / sec / 1e9 / HBM_PEAK_GBS,
            "mfma_frac": algorithmic_flops(wl) / sec / 1e12 / MFMA_PEAK_TFLOPS,
            "algorithmic_bytes_per_launch": algorithmic_bytes(wl), "kernel": kernel_desc(wl)}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--decode-steps", type=int, default=1000)
    ap.add_argument("--cpu-tokens", type=int, default=16384,
                    help="tokens per head of the oracle's sample (default %(default)s)")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-extra", action="store_true", help="skip the other prefill workloads")
    ap.add_argument("--backward", action="store_true",
                    help="time the gradient call (dr_chunk_bwd) on the main workload")
    ap.add_argument("--backward-workload", default="gdn_scalar_bf16_t4k",
                    help="workload of the gradient call's timing (default: %(default)s)")
    ap.add_argument("--no-backward", action="store_true", help="skip the gradient call's timing")
    ap.add_argument("--workload", default=PREFILL,
                    help="prefill workload of the main line (default: %(default)s)")
    ap.add_argument("--segment-scan", type=int, default=0, metavar="P",
                    help="also time the segment-parallel scan composed from dr_chunk_fwd_varlen (sliced "
                         "scans) with P segments per head on the main workload (design record only)")
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
    torch.cuda.empty_cache()
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
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic, "kernel": kernel_desc(wl),
                     "algorithmic_bytes_per_launch": nbytes},
        "mfma": {"achieved_tflops": flops / sec / 1e12, "peak_tflops": MFMA_PEAK_TFLOPS,
                 "frac": flops / sec / 1e12 / MFMA_PEAK_TFLOPS, "algorithmic_flops_per_launch": flops},
        "timed_wall_s": wall,
    }
    if not args.no_extra:
        extra = {}
        for name in EXTRA_PREFILL:
            if name == wl.name:
                continue
            w2 = workload(name)
            s2, _ = time_prefill(dr, torch, w2, max(5, args.steps // 5), 2)
            extra[name] = prefill_record(w2, s2)
            torch.cuda.empty_cache()
        line["other_prefill"] = extra
    if args.segment_scan:
        t_seg, t_one, rel = time_segment_scan(dr, torch, wl, args.segment_scan)
        line["segment_scan"] = {"segments": args.segment_scan, "ms": t_seg, "single_pass_ms": t_one,
                                "max_rel_diff": rel}
        torch.cuda.empty_cache()
    if not args.no_backward:
        bwl = wl if args.backward else workload(args.backward_workload)
        bsteps = max(5, args.steps // 10)
        bsec = time_backward(dr, torch, bwl, bsteps, 2)
        bbytes = backward_bytes(bwl)
        chunked = bwl.qkv_dtype == "bf16" and bwl.dk == 128 and bwl.dv == 128 and not bwl.seq_median
        line["backward"] = {"workload": bwl.name, "calls": bsteps, "ms": bsec * 1e3,
                            "tokens_per_s": bwl.token_heads / bsec,
                            "hbm_frac": bbytes / bsec / 1e9 / HBM_PEAK_GBS, "bytes_per_call": bbytes,
                            "kernel": ("dr_chunk_bwd = chunked forward (stores S and M or delta) + adjoint scan "
                                       "(stores G, Z) + chunk_grad_kernel + chunk_grad_sums_kernel")
                                      if chunked else
                                      "dr_chunk_bwd = bwd_token_kernel + bwd_reduce_kernel (fp32 token adjoint)"}
        if chunked:
            tsec = time_backward(dr, torch, bwl, 2, 1, chunk=1)
            line["backward"]["token_adjoint_ms"] = tsec * 1e3
            line["backward"]["speedup_over_token_adjoint"] = tsec / bsec
        if not args.no_cpu:
            line["backward"]["cpu_baseline"] = cpu_baseline_backward(bwl, max(64, args.cpu_tokens // 64))
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
