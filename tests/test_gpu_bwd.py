"""GPU parity of the gradients (dr_chunk_bwd) against the fp64 adjoint oracle.

Two paths.  The token path (fp32 q/k/v, other widths, packed sequences, or chunk = 1) evaluates
the adjoint of the token loop in fp32 from an fp32 forward, so its bar is the fp32 one:
normwise error (max |x - ref| / max |ref| per tensor) at most 1e-5.  The chunk path (bf16 q/k/v,
dk == dv == 128, a dense batch) starts every chunk's token adjoint from the state the
matrix-core forward stored at the chunk's start and from the adjoint the matrix-core adjoint
scan stored at its end, both computed with fp16 operands, so its bar is the forward's: 3e-3."""
import numpy as np
import pytest
import torch

from oracle import recurrence_bwd, recurrence_fg2_bwd

pytestmark = pytest.mark.gpu

TOL = 1e-5
TOL_CHUNK = 3e-3


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


def _check(dr, inp, dO, dST, with_dst=True, chunk=64):
    d = {k: (None if v is None else v.cuda()) for k, v in inp.items()}
    g = dr.chunk_bwd(d["q"], d["k"], d["v"], d["log_decay"], d["erase"], d["write"], d["S0"],
                     dO=dO.cuda(), dS_T=dST.cuda() if with_dst else None, chunk=chunk)
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


@pytest.mark.parametrize("chunk", [64, 1])
@pytest.mark.parametrize("T", [1, 63, 64, 65, 130, 300])
@pytest.mark.parametrize("variant", ["scalar", "kda", "decoupled"])
def test_bwd_variants_d128(dr, T, variant, chunk):
    inp, dO, dST = _case(2, T, 2, 128, 128, "bf16", variant, T % 2 == 1, 200 + T)
    errs = _check(dr, inp, dO, dST, chunk=chunk)
    print(f"bwd {variant} T={T} chunk={chunk}: " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    assert max(errs.values()) <= (TOL_CHUNK if chunk == 64 else TOL), errs


@pytest.mark.parametrize("T", [394, 520])
def test_bwd_segmented_scans(dr, T):
    # separate erase and write gates over a dense batch: both full-width scans (the forward with
    # its checkpoints and the adjoint) cut 2 x 2 heads of 7 and 9 chunks into 3 and 4 segments, so
    # the maps, the compose step in both directions and the entering states all take part
    from chunk_model import wide_plan

    assert wide_plan(4, T)[0] == (3 if T == 394 else 4)
    inp, dO, dST = _case(2, T, 2, 128, 128, "bf16", "decoupled", True, 700 + T)
    errs = _check(dr, inp, dO, dST)
    print(f"bwd segmented T={T}: " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    assert max(errs.values()) <= TOL_CHUNK, errs


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
    assert max(errs.values()) <= (TOL_CHUNK if d == 128 else TOL), errs


@pytest.mark.parametrize("chunk", [64, 1])
@pytest.mark.parametrize("variant", ["scalar", "kda", "decoupled"])
def test_bwd_packed_sequences(dr, variant, chunk):
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
                       dS_T=dST.cuda(), cu_seqlens=torch.tensor(cu, dtype=torch.int32, device="cuda"), chunk=chunk)
    torch.cuda.synchronize()
    tol = TOL_CHUNK if chunk == 64 else TOL
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
                assert _err(out[key][:, lo:hi], ref[key]) <= tol, (n, key)
        assert _err(out["dS0"][n:n + 1], ref["dS0"]) <= tol, n


@pytest.mark.parametrize("variant", ["scalar", "kda", "decoupled"])
def test_bwd_chunk_path_strong_decay(dr, variant):
    # strong decays, a ~ 0.5 per token (sigmoid(N(0, 1.5)) for the scalar gate,
    # exp(-softplus(N(0, 1.5))) per channel): the chunk path keeps its bar there too
    from gated_delta_rule_dr_amd.workloads import Workload, generate

    wl = Workload("case", 1, 200, 2, 128, 128, "bf16", "sigmoid" if variant == "scalar" else "softplus",
                  variant != "scalar", 0.0, 1.5, variant == "decoupled", "channel" if variant == "decoupled" else "erase",
                  0.05, 700)
    inp = generate(wl)
    g = torch.Generator().manual_seed(701)
    dO = torch.randn((1, 200, 2, 128), generator=g, dtype=torch.float64).float()
    dST = torch.randn((1, 2, 128, 128), generator=g, dtype=torch.float64).float()
    errs = _check(dr, inp, dO, dST)
    print(f"bwd strong decay {variant}: " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    assert max(errs.values()) <= TOL_CHUNK, errs


def test_bwd_full_shape_sampled_heads(dr):
    # the scalar-gate workload's shape (B4 H16 T4096) through the chunk path; the oracle checks
    # two (b, h) pairs over the whole sequence from the same inputs
    from gated_delta_rule_dr_amd.workloads import generate, workload

    wl = workload("gdn_scalar_bf16_t4k")
    inp = generate(wl, device="cuda")
    g = torch.Generator(device="cuda").manual_seed(702)
    dO = torch.randn((wl.B, wl.T, wl.H, wl.dv), generator=g, device="cuda")
    dST = torch.randn((wl.B, wl.H, wl.dk, wl.dv), generator=g, device="cuda")
    out = dr.chunk_bwd(inp["q"], inp["k"], inp["v"], inp["log_decay"], inp["erase"], inp["write"], inp["S0"],
                       dO=dO, dS_T=dST)
    torch.cuda.synchronize()
    for b, h in ((0, 0), (3, 15)):
        cut = lambda x: None if x is None else x[b:b + 1, :, h:h + 1].cpu()
        ref = recurrence_bwd(cut(inp["q"]), cut(inp["k"]), cut(inp["v"]), cut(inp["log_decay"]), cut(inp["erase"]),
                             cut(inp["write"]), None if inp["S0"] is None else inp["S0"][b:b + 1, h:h + 1].cpu(),
                             dO=cut(dO), dS_T=dST[b:b + 1, h:h + 1].cpu())
        errs = {}
        for key in ("dq", "dk", "dv", "dlog_decay", "derase"):
            errs[key] = _err(out[key][b:b + 1, :, h:h + 1], ref[key])
        errs["dS0"] = _err(out["dS0"][b:b + 1, h:h + 1], ref["dS0"])
        print(f"bwd full shape (b={b}, h={h}): " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()), flush=True)
        assert max(errs.values()) <= TOL_CHUNK, (b, h, errs)


@pytest.mark.parametrize("name, heads", [("kda_channel_bf16_t16k", ((0, 0), (1, 31))),
                                         ("gdn2_decoupled_bf16_t64k", ((0, 17),))])
def test_bwd_full_shape_long(dr, name, heads):
    # the KDA workload (B2 H32 T16384) and the long-context decoupled workload (B1 H32 T65536) at
    # full size through the chunk path; the oracle follows the sampled heads over the whole sequence
    from gated_delta_rule_dr_amd.workloads import generate, workload

    wl = workload(name)
    print(f"bwd full shape {name}", flush=True)
    inp = generate(wl, device="cuda")
    g = torch.Generator(device="cuda").manual_seed(703)
    dO = torch.randn((wl.B, wl.T, wl.H, wl.dv), generator=g, device="cuda")
    dST = torch.randn((wl.B, wl.H, wl.dk, wl.dv), generator=g, device="cuda")
    out = dr.chunk_bwd(inp["q"], inp["k"], inp["v"], inp["log_decay"], inp["erase"], inp["write"], inp["S0"],
                       dO=dO, dS_T=dST)
    torch.cuda.synchronize()
    for b, h in heads:
        cut = lambda x: None if x is None else x[b:b + 1, :, h:h + 1].cpu()
        ref = recurrence_bwd(cut(inp["q"]), cut(inp["k"]), cut(inp["v"]), cut(inp["log_decay"]), cut(inp["erase"]),
                             cut(inp["write"]), None if inp["S0"] is None else inp["S0"][b:b + 1, h:h + 1].cpu(),
                             dO=cut(dO), dS_T=dST[b:b + 1, h:h + 1].cpu())
        errs = {}
        for key in ("dq", "dk", "dv", "dlog_decay", "derase", "dwrite"):
            if ref[key] is None:
                assert out[key] is None
                continue
            errs[key] = _err(out[key][b:b + 1, :, h:h + 1], ref[key])
        errs["dS0"] = _err(out["dS0"][b:b + 1, h:h + 1], ref["dS0"])
        print(f"bwd full shape {name} (b={b}, h={h}): " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()),
              flush=True)
        assert max(errs.values()) <= TOL_CHUNK, (name, b, h, errs)


@pytest.mark.parametrize("variant", ["scalar", "kda", "decoupled", "fg2"])
@pytest.mark.parametrize("edge", ["no_decay", "no_erase", "full_gates"])
def test_bwd_chunk_path_edge_gates(dr, variant, edge):
    # log a = 0; erase = 0 (one gate: no write either, so the reads M come only from the state;
    # decoupled gates: gated linear attention); erase = write = 1
    fg2 = variant == "fg2"
    if fg2 and edge == "no_erase":
        pytest.skip("FG2's rate is a square root of beta > 0")
    inp, dO, dST = _case(1, 150, 2, 128, 128, "bf16", "kda" if fg2 else variant, True, 900)
    if fg2:
        from gated_delta_rule_dr_amd.workloads import Workload, generate

        wl = Workload("case", 1, 150, 2, 128, 128, "bf16", "softplus", True, -4.0, 1.5, True, "erase", 0.05, 901,
                      rate_sqrt=True)
        inp = generate(wl)
    if edge == "no_decay":
        inp["log_decay"] = torch.zeros_like(inp["log_decay"])
    elif edge == "no_erase":
        inp["erase"] = torch.zeros_like(inp["erase"])
    else:
        inp["erase"] = torch.ones_like(inp["erase"])
        if inp["write"] is not None:
            inp["write"] = torch.ones_like(inp["write"])
    if fg2:
        x = {k: (None if v is None else v.cuda()) for k, v in inp.items()}
        out = dr.chunk_bwd(x["q"], x["k"], x["v"], x["log_decay"], x["erase"], None, x["S0"], dO=dO.cuda(),
                           dS_T=dST.cuda(), fg2=True)
        torch.cuda.synchronize()
        ref = recurrence_fg2_bwd(inp["q"], inp["k"], inp["v"], inp["log_decay"], inp["erase"], inp["S0"], dO, dST)
        errs = {key: _err(out[key], ref[key]) for key in ("dq", "dk", "dv", "dlog_decay", "dS0")}
        errs["dbeta"] = _err(out["derase"], ref["dbeta"])
    else:
        errs = _check(dr, inp, dO, dST)
    print(f"bwd edge {variant} {edge}: " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    assert max(errs.values()) <= TOL_CHUNK, errs


def test_bwd_packed_fg2_rate(dr):
    # FG2's rate over packed sequences (one empty): each sequence's gradients against the rate
    # form's adjoint over its own tokens from its own state
    from gated_delta_rule_dr_amd.workloads import Workload, generate

    lens = [90, 0, 1, 130]
    T = sum(lens)
    wl = Workload("case", 1, T, 2, 128, 128, "bf16", "softplus", True, -4.0, 1.5, True, "erase", 0.0, 610,
                  rate_sqrt=True)
    inp = generate(wl)
    g = torch.Generator().manual_seed(611)
    N = len(lens)
    S0 = (0.05 * torch.randn((N, 2, 128, 128), generator=g, dtype=torch.float64)).float()
    dO = torch.randn((1, T, 2, 128), generator=g, dtype=torch.float64).float()
    dST = torch.randn((N, 2, 128, 128), generator=g, dtype=torch.float64).float()
    cu = np.concatenate([[0], np.cumsum(lens)])
    x = {k: (None if v is None else v.cuda()) for k, v in inp.items()}
    out = dr.chunk_bwd(x["q"], x["k"], x["v"], x["log_decay"], x["erase"], None, S0.cuda(), dO=dO.cuda(),
                       dS_T=dST.cuda(), fg2=True, cu_seqlens=torch.tensor(cu, dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    for n in range(N):
        lo, hi = int(cu[n]), int(cu[n + 1])
        if hi == lo:
            assert torch.equal(out["dS0"][n].cpu(), dST[n])
            continue
        cut = lambda key: inp[key][:, lo:hi]
        ref = recurrence_fg2_bwd(cut("q"), cut("k"), cut("v"), cut("log_decay"), cut("erase"), S0[n:n + 1],
                                 dO[:, lo:hi], dST[n:n + 1])
        for key in ("dq", "dk", "dv", "dlog_decay"):
            assert _err(out[key][:, lo:hi], ref[key]) <= TOL_CHUNK, (n, key)
        assert _err(out["derase"][:, lo:hi], ref["dbeta"]) <= TOL_CHUNK, n
        assert _err(out["dS0"][n:n + 1], ref["dS0"]) <= TOL_CHUNK, n
