"""The allocation-free forward (dr_chunk_fwd_noalloc) against dr_chunk_fwd, through the C ABI.

The two entry points run the same kernels; the allocation-free one takes its workspace from the
library's fixed device scratch.  Two calls in a row (the second on a smaller problem, so that it
reads a scratch that still holds the first call's larger contents) must give results identical
to dr_chunk_fwd's, element by element, and a problem larger than the scratch must be refused
before any device work.
"""
import ctypes

import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dr():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gated_delta_rule_dr_amd as m

    m.abi_version()
    return m


def _inputs(variant, B, T, H, seed):
    from gated_delta_rule_dr_amd.workloads import Workload, generate

    wl = Workload("case", B, T, H, 128, 128, "bf16", "softplus", variant != "scalar", -2.0, 1.5,
                  variant == "decoupled", "channel" if variant == "decoupled" else "erase", 0.05, seed)
    return {k: (None if v is None else v.cuda()) for k, v in generate(wl).items()}


def _both(dr, x):
    o_ref, S_ref = dr.chunk_fwd(x["q"], x["k"], x["v"], x["log_decay"], x["erase"], x["write"], x["S0"])
    o = torch.full_like(o_ref, float("nan"))
    S = torch.full_like(S_ref, float("nan"))
    dr.chunk_fwd_noalloc(x["q"], x["k"], x["v"], x["log_decay"], x["erase"], x["write"], x["S0"], out=o, S_T=S)
    torch.cuda.synchronize()
    return o, S, o_ref, S_ref


@pytest.mark.parametrize("variant", ["scalar", "kda", "decoupled"])
def test_noalloc_matches_chunk_fwd_two_calls(dr, variant):
    # first call: 2 x 8 heads x 520 tokens; second: 1 x 3 heads x 130 tokens
    for B, T, H, seed in ((2, 520, 8, 11), (1, 130, 3, 12)):
        x = _inputs(variant, B, T, H, seed)
        o, S, o_ref, S_ref = _both(dr, x)
        print(f"{variant} B={B} T={T} H={H}: equal o={torch.equal(o, o_ref)} S={torch.equal(S, S_ref)}")
        assert torch.equal(o, o_ref) and torch.equal(S, S_ref)


def test_noalloc_token_path_and_empty(dr):
    # fp32 inputs take the token-by-token path (no workspace); T = 0 copies S0
    x = _inputs("kda", 1, 37, 2, 13)
    xf = dict(x, q=x["q"].float(), k=x["k"].float(), v=x["v"].float())
    o, S, o_ref, S_ref = _both(dr, xf)
    assert torch.equal(o, o_ref) and torch.equal(S, S_ref)
    e = _inputs("kda", 1, 0, 2, 14)
    o = torch.empty((1, 0, 2, 128), device="cuda")
    S = torch.full((1, 2, 128, 128), 7.0, device="cuda")
    dr.chunk_fwd_noalloc(e["q"], e["k"], e["v"], e["log_decay"], e["erase"], None, e["S0"], out=o, S_T=S)
    torch.cuda.synchronize()
    assert torch.equal(S, e["S0"])


def test_noalloc_refuses_problems_beyond_its_scratch(dr):
    from gated_delta_rule_dr_amd import _abi

    cap = dr.noalloc_max_bytes()
    assert cap == 64 << 20
    # 64 heads x 1,600 tokens of per-channel gates need 1,600 chunks x 92,160 B > 64 MiB
    B, T, H = 1, 1600, 64
    x = _inputs("decoupled", B, T, H, 15)
    o = torch.full((B, T, H, 128), 3.0, device="cuda")
    with pytest.raises(_abi.DrError) as ei:
        dr.chunk_fwd_noalloc(x["q"], x["k"], x["v"], x["log_decay"], x["erase"], x["write"], x["S0"], out=o)
    assert ei.value.status == _abi.DR_E_SCRATCH
    torch.cuda.synchronize()
    assert bool((o == 3.0).all())  # nothing was enqueued
