"""GPU parity of the gradients (dr_chunk_bwd) against the fp64 adjoint oracle.

The kernels evaluate the adjoint of the token loop in fp32 (with the bf16 or fp32 inputs as
stored), so the bar is the fp32 one: normwise error (max |x - ref| / max |ref| per tensor)
at most 1e-5 over sequences of a few hundred tokens."""
import numpy as np
import pytest
import torch

from oracle import recurrence_bwd, recurrence_fg2_bwd

pytestmark = pytest.mark.gpu

TOL = 1e-5


@pytest.fixture(scope="module")
def dr():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gated_delta_rule_dr_amd as m

    m.abi_version()
    return m


def _case(B, T, H, dk, dv, dtype, variant, s0, seed):
    from gated_delta_rule_dr_amd.workloads import Workload, generate

    decay_ch = variant != "scalar"
    erase_ch = variant in ("decoupled", "channel_shared")
    write = "channel" if variant == "decoupled" else "erase"
    wl = Workload("case", B, T, H, dk, dv, dtype, "softplus", decay_ch, -4.0, 1.5, erase_ch, write,
                  0.05 if s0 else 0.0, seed)
    inp = generate(wl)
    g = torch.Generator().manual_seed(seed + 7)
    dO = torch.randn((B, T, H, dv), generator=g, dtype=torch.float64).float()
    dST = torch.randn((B, H, dk, dv), generator=g, dtype=torch.float64).float()
    return inp, dO, dST


def _err(x, ref):
    x = x.double().cpu().numpy()
    den = np.abs(ref).max()
    return float(np.abs(x - ref).max() / (den if den > 0 else 1.0))


def _check(dr, inp, dO, dST, with_dst=True):
    d = {k: (None if v is None else v.cuda()) for k, v in inp.items()}
    g = dr.chunk_bwd(d["q"], d["k"], d["v"], d["log_decay"], d["erase"], d["write"], d["S0"],
                     dO=dO.cuda(), dS_T=dST.cuda() if with_dst else None)
    torch.cuda.synchronize()
    ref = recurrence_bwd(inp["q"], inp["k"], inp["v"], inp["log_decay"], inp["erase"], inp["write"], inp["S0"],
                         dO=dO, dS_T=dST if with_dst else None)
    errs = {}
    for key in ("dq", "dk", "dv", "dlog_decay", "derase", "dwrite", "dS0"):
        if ref[key] is None:
            assert g[key] is None
            continue
        errs[key] = _err(g[key], ref[key])
    return errs


@pytest.mark.parametrize("T", [1, 63, 64, 65, 130])
@pytest.mark.parametrize("variant", ["scalar", "kda", "decoupled"])
def test_bwd_variants_d128(dr, T, variant):
    inp, dO, dST = _case(2, T, 2, 128, 128, "bf16", variant, T % 2 == 1, 200 + T)
    errs = _check(dr, inp, dO, dST)
    print(f"bwd {variant} T={T}: " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    assert max(errs.values()) <= TOL, errs


@pytest.mark.parametrize("dk,dv", [(16, 16), (32, 64), (64, 32)])
@pytest.mark.parametrize("variant", ["scalar", "decoupled"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_bwd_widths(dr, dk, dv, variant, dtype):
    inp, dO, dST = _case(1, 70, 3, dk, dv, dtype, variant, True, 300 + dk + dv)
    errs = _check(dr, inp, dO, dST)
    assert max(errs.values()) <= TOL, errs


def test_bwd_shared_channel_gate_and_no_dst(dr):
    # one per-channel gate for erase and write (dk == dv): its gradient has both parts
    inp, dO, dST = _case(1, 100, 2, 64, 64, "bf16", "channel_shared", True, 400)
    errs = _check(dr, inp, dO, dST, with_dst=False)
    assert max(errs.values()) <= TOL, errs


def test_bwd_zero_length(dr):
    inp, dO, dST = _case(2, 0, 2, 128, 128, "bf16", "kda", True, 401)
    d = {k: (None if v is None else v.cuda()) for k, v in inp.items()}
    g = dr.chunk_bwd(d["q"], d["k"], d["v"], d["log_decay"], d["erase"], d["write"], d["S0"],
                     dO=dO.cuda(), dS_T=dST.cuda())
    torch.cuda.synchronize()
    assert torch.equal(g["dS0"].cpu(), dST)


def test_bwd_deterministic(dr):
    inp, dO, dST = _case(2, 90, 2, 128, 128, "bf16", "decoupled", True, 402)
    d = {k: (None if v is None else v.cuda()) for k, v in inp.items()}
    run = lambda: dr.chunk_bwd(d["q"], d["k"], d["v"], d["log_decay"], d["erase"], d["write"], d["S0"],
                               dO=dO.cuda(), dS_T=dST.cuda())
    a, b = run(), run()
    torch.cuda.synchronize()
    for key in a:
        if a[key] is not None:
            assert torch.equal(a[key], b[key]), key


@pytest.mark.parametrize("decay_channel", [True, False])
@pytest.mark.parametrize("d", [64, 128])
def test_bwd_fg2_rate(dr, decay_channel, d):
    from gated_delta_rule_dr_amd.workloads import Workload, generate

    wl = Workload("case", 1, 90, 2, d, d, "bf16", "softplus", decay_channel, -4.0, 1.5, True, "erase", 0.05, 500 + d,
                  rate_sqrt=True)
    inp = generate(wl)
    g = torch.Generator().manual_seed(501)
    dO = torch.randn((1, 90, 2, d), generator=g, dtype=torch.float64).float()
    dST = torch.randn((1, 2, d, d), generator=g, dtype=torch.float64).float()
    x = {k: (None if v is None else v.cuda()) for k, v in inp.items()}
    out = dr.chunk_bwd(x["q"], x["k"], x["v"], x["log_decay"], x["erase"], None, x["S0"], dO=dO.cuda(),
                       dS_T=dST.cuda(), fg2=True)
    torch.cuda.synchronize()
    ref = recurrence_fg2_bwd(inp["q"], inp["k"], inp["v"], inp["log_decay"], inp["erase"], inp["S0"], dO, dST)
    errs = {key: _err(out[key], ref[key]) for key in ("dq", "dk", "dv", "dlog_decay", "dS0")}
    errs["dbeta"] = _err(out["derase"], ref["dbeta"])
    assert max(errs.values()) <= TOL, errs


@pytest.mark.parametrize("variant", ["scalar", "decoupled"])
def test_bwd_packed_sequences(dr, variant):
    # packed sequences (one empty, ragged lengths): each sequence's gradients equal the dense
    # adjoint over its own tokens from its own state
    lens = [70, 0, 1, 129, 64]
    inp, dO, _ = _case(1, sum(lens), 2, 128, 128, "bf16", variant, False, 600)
    g = torch.Generator().manual_seed(601)
    N = len(lens)
    S0 = (0.05 * torch.randn((N, 2, 128, 128), generator=g, dtype=torch.float64)).float()
    dST = torch.randn((N, 2, 128, 128), generator=g, dtype=torch.float64).float()
    cu = np.concatenate([[0], np.cumsum(lens)])
    x = {k: (None if v is None else v.cuda()) for k, v in inp.items()}
    out = dr.chunk_bwd(x["q"], x["k"], x["v"], x["log_decay"], x["erase"], x["write"], S0.cuda(), dO=dO.cuda(),
                       dS_T=dST.cuda(), cu_seqlens=torch.tensor(cu, dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    for n in range(N):
        lo, hi = int(cu[n]), int(cu[n + 1])
        if hi == lo:
            assert torch.equal(out["dS0"][n].cpu(), dST[n])
            continue
        cut = lambda key: None if inp[key] is None else inp[key][:, lo:hi]
        ref = recurrence_bwd(cut("q"), cut("k"), cut("v"), cut("log_decay"), cut("erase"), cut("write"), S0[n:n + 1],
                             dO=dO[:, lo:hi], dS_T=dST[n:n + 1])
        for key in ("dq", "dk", "dv", "dlog_decay", "derase", "dwrite"):
            if ref[key] is not None:
                assert _err(out[key][:, lo:hi], ref[key]) <= TOL, (n, key)
        assert _err(out["dS0"][n:n + 1], ref["dS0"]) <= TOL, n
