"""Seeded synthetic inputs for the gated delta-rule hot path.

This module draws random numbers and shapes them into the gate parameterisations; it holds
none of the recurrence's arithmetic.  The same tensors feed the HIP path (through the
binding) and the fp64 oracle, so both sides always see identical values.

Recipe (numbers, dtypes and draw order), per workload:
  * draw order: q, k, v, decay noise, erase noise, write noise, then S0; each tensor in C order
    of its [B, T, H, d] (or [B, T, H]) layout.  Decode workloads draw S0 first and then every
    step's inputs stacked step-major: q[steps, N, H, dk], k, v, decay, erase.
  * q, k, v ~ N(0, 1); k is L2-normalised per token in fp64 before rounding.
  * decay: "sigmoid"    alpha = sigmoid(N(mu, sd)) passed as log alpha = -softplus(-x);
           "softplus"   log a = -softplus(N(mu, sd)).   sd is a standard deviation.
  * erase / write gates: sigmoid(N(0, 1)).
  * S0 ~ N(0, s0_std) when s0_std > 0, else no initial state (zeros).
  * packed workloads (seq_median > 0): B == 1 and the T tokens are split into sequences whose
    lengths are drawn first, from their own generator seeded with seed + 7919, as
    round(exp(log(seq_median) + N(0, 1))) clipped to [1, seq_max], until they cover T (the last
    one is cut to fit); cu_seqlens are their offsets and S0 is [N, H, dk, dv].
  * gates and S0 are computed in fp64 and rounded to fp32 (round to nearest even); q, k, v are
    rounded to bf16 (round to nearest even) for the bf16 workloads.
On the CPU the generator is torch's CPU generator; ``device="cuda"`` draws on the GPU with
torch's device generator (different random streams, same distributions) so that the
multi-GiB workloads can be built in seconds.
"""
from __future__ import annotations

import dataclasses
import math
from dataclasses import dataclass

import torch

__all__ = ["Workload", "WORKLOADS", "generate", "generate_decode", "seq_lengths", "workload"]


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    T: int
    H: int
    dk: int
    dv: int
    qkv_dtype: str  # "f32" | "bf16"
    decay: str  # "sigmoid" | "softplus"
    decay_channel: bool  # per-channel [.., dk] decay instead of one scalar per head
    decay_mu: float
    decay_sd: float
    erase_channel: bool  # per-channel erase gate [.., dk]
    write: str  # "erase" (write gate == erase gate) | "channel" (own per-channel gate [.., dv])
    s0_std: float
    seed: int
    chunk: int = 64
    steps: int = 0  # decode workloads: number of single-token steps
    seq_median: int = 0  # packed workloads: median sequence length (0: a dense [B, T] batch)
    seq_max: int = 0  # packed workloads: longest sequence
    rate_sqrt: bool = False  # the per-channel erase gate is FG2-GDN's rate beta (sqrt into k and v)

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)

    @property
    def token_heads(self) -> int:
        return self.B * self.T * self.H


# The five workloads.  Context lengths follow those the pages evaluate (4k-16k, 32k+ for the
# long-context scaling claim); the shapes are the ones the build is measured on.
WORKLOADS = {
    w.name: w
    for w in [
        # scalar-gate Gated DeltaNet, fp32 throughout, small parity case
        Workload("gdn_scalar_f32_d32", 1, 256, 2, 32, 32, "f32", "sigmoid", False, 3.0, 1.0,
                 False, "erase", 0.0, 1),
        # scalar-gate Gated DeltaNet prefill, bf16 q/k/v, fp32 gates and state
        Workload("gdn_scalar_bf16_t4k", 4, 4096, 16, 128, 128, "bf16", "softplus", False, -4.0,
                 1.0, False, "erase", 0.0, 2),
        # KDA channel-wise decay prefill
        Workload("kda_channel_bf16_t16k", 2, 16384, 32, 128, 128, "bf16", "softplus", True,
                 -4.0, 1.5, False, "erase", 0.0, 3),
        # decoupled per-channel erase / write (Gated DeltaNet-2, FG2-GDN+) long-context prefill
        Workload("gdn2_decoupled_bf16_t64k", 1, 65536, 32, 128, 128, "bf16", "softplus", True,
                 -4.0, 1.5, True, "channel", 0.0, 4),
        # FG2-GDN prefill at the KDA workload's shape: channel decay and a per-channel rate
        # beta = sigmoid(N(0, 1)) absorbed as sqrt(beta) into k and v
        Workload("fg2_channel_bf16_t16k", 2, 16384, 32, 128, 128, "bf16", "softplus", True, -4.0,
                 1.5, True, "erase", 0.0, 7, rate_sqrt=True),
        # serving prefill: scalar-gate Gated DeltaNet over 16384 packed tokens of sequences of
        # mixed lengths (median 512, at most 4096), 16 heads
        Workload("gdn_scalar_bf16_varlen_t16k", 1, 16384, 16, 128, 128, "bf16", "softplus", False,
                 -4.0, 1.0, False, "erase", 0.0, 6, seq_median=512, seq_max=4096),
        # single-token decode, 256 sequences x 32 heads, resident fp32 state
        Workload("decode_kda_n256_h32", 256, 1, 32, 128, 128, "bf16", "softplus", True, -4.0,
                 1.5, False, "erase", 0.01, 5, steps=1000),
    ]
}


def workload(name: str, **overrides) -> Workload:
    wl = WORKLOADS[name]
    return wl.replace(**overrides) if overrides else wl


def _normal(gen, shape, device):
    return torch.randn(shape, generator=gen, device=device, dtype=torch.float64)


def _qkv_round(x, qkv_dtype):
    return x.to(torch.bfloat16) if qkv_dtype == "bf16" else x.to(torch.float32)


def _log_decay(gen, wl, lead, device):
    shape = lead + ((wl.dk,) if wl.decay_channel else ())
    x = wl.decay_mu + wl.decay_sd * _normal(gen, shape, device)
    if wl.decay == "sigmoid":  # alpha = sigmoid(x)  =>  log alpha = -softplus(-x)
        la = -torch.nn.functional.softplus(-x)
    elif wl.decay == "softplus":
        la = -torch.nn.functional.softplus(x)
    else:
        raise ValueError(wl.decay)
    return la.to(torch.float32)


def _sigmoid_gate(gen, shape, device):
    return torch.sigmoid(_normal(gen, shape, device)).to(torch.float32)


def _unit_rows(x):
    return x / torch.linalg.vector_norm(x, dim=-1, keepdim=True)


def seq_lengths(wl: Workload) -> list[int]:
    """Sequence lengths of a packed workload (see the recipe above); they sum to wl.T."""
    gen = torch.Generator()
    gen.manual_seed(wl.seed + 7919)
    lens, total = [], 0
    while total < wl.T:
        x = float(torch.randn((), generator=gen, dtype=torch.float64))
        n = min(max(round(math.exp(math.log(wl.seq_median) + x)), 1), wl.seq_max, wl.T - total)
        lens.append(n)
        total += n
    return lens


def generate(wl: Workload, device="cpu", value_seed=None):
    """Inputs for one prefill call: dict with q, k, v, log_decay, erase, write (or None), S0
    (or None), all in the [B, T, H, d] layout the library takes; packed workloads add
    cu_seqlens (int32 [N + 1], on ``device``) and take S0 as [N, H, dk, dv].  ``value_seed``
    (default wl.seed) seeds the values only; packed sequence lengths always follow wl.seed."""
    gen = torch.Generator(device=device)
    gen.manual_seed(wl.seed if value_seed is None else value_seed)
    lead = (wl.B, wl.T, wl.H)
    q = _qkv_round(_normal(gen, lead + (wl.dk,), device), wl.qkv_dtype)
    k = _qkv_round(_unit_rows(_normal(gen, lead + (wl.dk,), device)), wl.qkv_dtype)
    v = _qkv_round(_normal(gen, lead + (wl.dv,), device), wl.qkv_dtype)
    log_decay = _log_decay(gen, wl, lead, device)
    erase = _sigmoid_gate(gen, lead + ((wl.dk,) if wl.erase_channel else ()), device)
    write = _sigmoid_gate(gen, lead + (wl.dv,), device) if wl.write == "channel" else None
    nstate = wl.B
    extra = {}
    if wl.seq_median > 0:
        if wl.B != 1:
            raise ValueError("packed workloads have B == 1")
        lens = seq_lengths(wl)
        nstate = len(lens)
        cu = torch.zeros(nstate + 1, dtype=torch.int32)
        cu[1:] = torch.cumsum(torch.tensor(lens, dtype=torch.int64), 0).to(torch.int32)
        extra["cu_seqlens"] = cu.to(device)
    S0 = None
    if wl.s0_std > 0:
        S0 = (wl.s0_std * _normal(gen, (nstate, wl.H, wl.dk, wl.dv), device)).to(torch.float32)
    return dict(q=q, k=k, v=v, log_decay=log_decay, erase=erase, write=write, S0=S0, **extra)


def generate_decode(wl: Workload, steps: int | None = None, device="cpu"):
    """Inputs for ``steps`` consecutive decode steps of ``wl`` (T must be 1).

    Returns dict with S0 [N, H, dk, dv] and step-stacked q, k, v [steps, N, H, d],
    log_decay [steps, N, H(, dk)], erase [steps, N, H(, dk)], write (or None)."""
    if wl.T != 1:
        raise ValueError("decode workloads have T == 1")
    steps = wl.steps if steps is None else steps
    gen = torch.Generator(device=device)
    gen.manual_seed(wl.seed)
    N, H = wl.B, wl.H
    S0 = (wl.s0_std * _normal(gen, (N, H, wl.dk, wl.dv), device)).to(torch.float32)
    lead = (steps, N, H)
    q = _qkv_round(_normal(gen, lead + (wl.dk,), device), wl.qkv_dtype)
    k = _qkv_round(_unit_rows(_normal(gen, lead + (wl.dk,), device)), wl.qkv_dtype)
    v = _qkv_round(_normal(gen, lead + (wl.dv,), device), wl.qkv_dtype)
    log_decay = _log_decay(gen, wl, lead, device)
    erase = _sigmoid_gate(gen, lead + ((wl.dk,) if wl.erase_channel else ()), device)
    write = _sigmoid_gate(gen, lead + (wl.dv,), device) if wl.write == "channel" else None
    return dict(S0=S0, q=q, k=k, v=v, log_decay=log_decay, erase=erase, write=write)
