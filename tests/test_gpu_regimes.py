"""GPU parity over the whole range of valid gates, through the C ABI, against the fp64 oracle.

The method allows any decay a in (0, 1), per channel or per head ("Gated DeltaNet-2", the
solution and its gate table: channel-level decay inherited from KDA; "FG2-GDN", section 2,
update rule with Diag(alpha_t)), and any erase/write strengths in [0, 1].  These cases sweep the
decay from weak (a ~ 0.98, the regime of the workloads) to extreme (log a ~ -40 per token), and
cover the gates' special cases: no decay, no erase (gated linear attention, "KronLSTM ...", The
problem), full erase and write with unit keys (exact memory: S_t^T k_t = v_t, "FG2-GDN" section 2,
the Householder structure), large values, and one head's NaN staying inside that head.

Tolerances (normwise per (b, h), tests/metrics.py): 3e-3 for the bf16 matrix-core chunk path,
1e-5 for the fp32 token-by-token path (chunk = 1).
"""
import numpy as np
import pytest
import torch

from metrics import err_S, err_o
from oracle import recurrence, recurrence_fg2

pytestmark = pytest.mark.gpu

TOL_F32 = 1e-5
TOL_BF16 = 3e-3


@pytest.fixture(scope="module")
def dr():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gated_delta_rule_dr_amd as m

    m.abi_version()
    return m


def _inputs(variant, decay, mu, sd, T, H, seed, s0=0.05):
    from gated_delta_rule_dr_amd.workloads import Workload, generate

    # decoupled_head: per-channel erase and write gates with a per-head decay
    wl = Workload("case", 1, T, H, 128, 128, "bf16", decay, variant not in ("scalar", "decoupled_head"), mu, sd,
                  variant in ("decoupled", "decoupled_head", "fg2"),
                  "channel" if variant.startswith("decoupled") else "erase", s0, seed, rate_sqrt=variant == "fg2")
    return generate(wl)


def _run(dr, inp, fg2=False, chunk=64):
    d = {k: (None if v is None else v.cuda()) for k, v in inp.items()}
    o, S = dr.chunk_fwd(d["q"], d["k"], d["v"], d["log_decay"], d["erase"], d["write"], d["S0"], chunk=chunk,
                        fg2=fg2)
    torch.cuda.synchronize()
    return o, S


def _oracle(inp, fg2=False):
    if fg2:
        return recurrence_fg2(inp["q"], inp["k"], inp["v"], inp["log_decay"], inp["erase"], inp["S0"])
    return recurrence(inp["q"], inp["k"], inp["v"], inp["log_decay"], inp["erase"], inp["write"], inp["S0"])


SCALAR_REGIMES = [("sigmoid", 3.0, 1.0), ("sigmoid", 1.0, 1.0), ("sigmoid", 0.0, 1.0), ("sigmoid", -1.0, 1.0)]
CHANNEL_REGIMES = [("softplus", -4.0, 1.5), ("softplus", -1.0, 1.5), ("softplus", 0.0, 1.5), ("softplus", 2.0, 1.5)]
CASES = ([(v,) + r for v in ("scalar", "decoupled_head") for r in SCALAR_REGIMES] +
         [(v,) + r for v in ("kda", "decoupled", "fg2") for r in CHANNEL_REGIMES])


@pytest.mark.parametrize("T,H", [(65, 2), (200, 2), (130, 64)])
@pytest.mark.parametrize("variant,decay,mu,sd", CASES)
def test_chunk_path_decay_regimes(dr, variant, decay, mu, sd, T, H):
    # H = 2 runs the scans' 16-column value slices, H = 64 the 32-column ones
    inp = _inputs(variant, decay, mu, sd, T, H, 100 + T + H)
    fg2 = variant == "fg2"
    o, S = _run(dr, inp, fg2)
    ro, rS = _oracle(inp, fg2)
    eo, eS = err_o(o, ro), err_S(S, rS)
    print(f"{variant} {decay}({mu},{sd}) T={T} H={H}: err_o={eo:.3e} err_S={eS:.3e}")
    assert eo <= TOL_BF16 and eS <= TOL_BF16, (eo, eS)


@pytest.mark.parametrize("variant,decay,mu,sd", [("scalar", "sigmoid", -1.0, 1.0), ("kda", "softplus", 2.0, 1.5),
                                                 ("decoupled", "softplus", 2.0, 1.5)])
def test_token_path_decay_regimes(dr, variant, decay, mu, sd):
    inp = _inputs(variant, decay, mu, sd, 100, 3, 7)
    o, S = _run(dr, inp, chunk=1)
    ro, rS = _oracle(inp)
    assert err_o(o, ro) <= TOL_F32 and err_S(S, rS) <= TOL_F32


@pytest.mark.parametrize("variant", ["scalar", "kda", "decoupled"])
def test_extreme_decay(dr, variant):
    # log a ~ -softplus(N(40, 10)): the state forgets within a token
    decay = "sigmoid" if variant == "scalar" else "softplus"
    inp = _inputs(variant, decay, -40.0 if variant == "scalar" else 40.0, 10.0, 200, 2, 9)
    o, S = _run(dr, inp)
    ro, rS = _oracle(inp)
    assert err_o(o, ro) <= TOL_BF16 and err_S(S, rS) <= TOL_BF16


def test_mixed_blocks_in_one_chunk(dr):
    # two strongly decaying 16-token blocks inside otherwise weak chunks: both splits of the
    # diagonal blocks in one chunk
    inp = _inputs("kda", "softplus", -4.0, 1.5, 200, 2, 5)
    hard = _inputs("kda", "softplus", 2.0, 1.5, 200, 2, 6)["log_decay"]
    inp["log_decay"][:, 64:96] = hard[:, 64:96]
    inp["log_decay"][:, 150:160] = hard[:, 150:160]
    o, S = _run(dr, inp)
    ro, rS = _oracle(inp)
    assert err_o(o, ro) <= TOL_BF16 and err_S(S, rS) <= TOL_BF16


@pytest.mark.parametrize("variant", ["scalar", "kda", "decoupled"])
@pytest.mark.parametrize("edge", ["no_decay", "no_erase", "full_gates", "large_v"])
def test_edge_gates(dr, variant, edge):
    # strong decay (a ~ 0.5), except without erase: with symmetric gates nothing is then written
    # and the state is S0 decayed below fp32's range over 150 tokens (checked separately below)
    weak = edge == "no_erase"
    scalar = variant == "scalar"
    inp = _inputs(variant, "sigmoid" if scalar else "softplus", (3.0 if scalar else -4.0) if weak else 0.0, 1.5,
                  150, 2, 21)
    if edge == "no_decay":
        inp["log_decay"] = torch.zeros_like(inp["log_decay"])
    elif edge == "no_erase":  # symmetric gates: no write either; decoupled: gated linear attention
        inp["erase"] = torch.zeros_like(inp["erase"])
    elif edge == "full_gates":
        inp["erase"] = torch.ones_like(inp["erase"])
        if inp["write"] is not None:
            inp["write"] = torch.ones_like(inp["write"])
    else:
        inp["v"] = (inp["v"].double() * 1000.0).to(torch.bfloat16)
    o, S = _run(dr, inp)
    ro, rS = _oracle(inp)
    eo, eS = err_o(o, ro), err_S(S, rS)
    print(f"{variant} {edge}: err_o={eo:.3e} err_S={eS:.3e}")
    assert eo <= TOL_BF16 and eS <= TOL_BF16, (eo, eS)


@pytest.mark.parametrize("variant", ["scalar", "kda"])
def test_no_write_state_decays_away(dr, variant):
    # symmetric gates with erase = 0 write nothing; under strong decay S0 decays below fp32's
    # range (true S_T ~ 1e-50): o and S_T are then zero up to fp32 underflow on both sides
    inp = _inputs(variant, "sigmoid" if variant == "scalar" else "softplus", 0.0, 1.5, 150, 2, 21)
    inp["erase"] = torch.zeros_like(inp["erase"])
    o, S = _run(dr, inp)
    ro, rS = _oracle(inp)
    assert float(np.abs(rS).max()) < 1e-30 and float(S.abs().max()) < 1e-30
    assert err_o(o, ro) <= TOL_BF16


def test_exact_memory_readback(dr):
    # unit keys, erase = write = 1, no decay: every step stores v_t exactly along k_t, so the
    # output read along the same key (q_t = k_t) returns v_t
    inp = _inputs("kda", "softplus", 0.0, 1.5, 130, 2, 33, s0=0.0)
    inp["log_decay"] = torch.zeros_like(inp["log_decay"])
    inp["erase"] = torch.ones_like(inp["erase"])
    inp["q"] = inp["k"].clone()
    o, S = _run(dr, inp)
    v = inp["v"].double()
    rel = float((o.cpu().double() - v).abs().max() / v.abs().max())
    assert rel <= TOL_BF16, rel


@pytest.mark.parametrize("variant", ["scalar", "kda", "decoupled"])
def test_nan_stays_in_its_head(dr, variant):
    # a NaN in one head's query poisons that head's outputs only; the other heads are bitwise
    # the same as in a clean run
    inp = _inputs(variant, "sigmoid" if variant == "scalar" else "softplus", -1.0, 1.5, 130, 4, 41)
    o_ref, S_ref = _run(dr, inp)
    bad = dict(inp)
    bad["q"] = inp["q"].clone()
    bad["q"][0, 70, 1, 5] = float("nan")
    bad["k"] = inp["k"].clone()
    bad["k"][0, 90, 2, 3] = float("nan")
    o, S = _run(dr, bad)
    for h in (0, 3):
        assert torch.equal(o[:, :, h], o_ref[:, :, h]) and torch.equal(S[:, h], S_ref[:, h])
    assert torch.isnan(o[:, 70:, 1]).any()
    assert torch.isnan(S[:, 2]).any()
