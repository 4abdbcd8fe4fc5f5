"""The matrix-core chunk path's referencing scheme, emulated in fp64 on the CPU (tests/chunk_model.py,
``kernel_emulation``), against the fp64 oracle over the whole range of valid decays.

The method allows any decay a in (0, 1) per channel or per head ("Gated DeltaNet-2", the solution
and its gate table: channel-level decay inherited from KDA; "FG2-GDN", section 2, update rule with
Diag(alpha_t)).  The kernel multiplies fp16 operands, so how each in-chunk factor e^{g_t - g_i} is
split between the two operands of a product decides whether the path is exact for every such
decay.  These tests fix that: the scheme the kernels implement ("safe") meets the bf16 parity bar
(3e-3, normwise) for scalar, KDA, decoupled and FG2 gates from weak to extreme decay, and the
first kernel's midpoint referencing, kept here as the planted mistake, fails once half a chunk's
log-decay passes -11.
"""
import numpy as np
import pytest

from chunk_model import kernel_emulation
from metrics import err_S, err_o
from oracle import recurrence, recurrence_fg2

TOL_BF16 = 3e-3


def _inputs(variant, decay, mu, sd, T=200, H=2, seed=1, s0=0.05, v_scale=1.0):
    from gated_delta_rule_dr_amd.workloads import Workload, generate

    wl = Workload("case", 1, T, H, 128, 128, "bf16", decay, variant != "scalar", mu, sd,
                  variant in ("decoupled", "fg2"), "channel" if variant == "decoupled" else "erase", s0, seed,
                  rate_sqrt=variant == "fg2")
    inp = generate(wl)
    if v_scale != 1.0:
        import torch

        inp["v"] = (inp["v"].double() * v_scale).to(torch.bfloat16)
    return inp


def _f(x):
    return None if x is None else x.double().numpy()


def _oracle(inp, fg2):
    if fg2:
        return recurrence_fg2(inp["q"], inp["k"], inp["v"], inp["log_decay"], inp["erase"], inp["S0"])
    return recurrence(inp["q"], inp["k"], inp["v"], inp["log_decay"], inp["erase"], inp["write"], inp["S0"])


def _emulate(inp, scheme, fg2):
    q, k, v = _f(inp["q"]), _f(inp["k"]), _f(inp["v"])
    B, T, H, _ = q.shape
    o = np.zeros(v.shape)
    S = np.zeros((B, H, k.shape[-1], v.shape[-1]))
    flags = []
    for h in range(H):
        sel = lambda x: None if x is None else _f(x)[0, :, h]
        s0 = None if inp["S0"] is None else _f(inp["S0"])[0, h]
        oo, SS, fl = kernel_emulation(sel(inp["q"]), sel(inp["k"]), sel(inp["v"]), sel(inp["log_decay"]),
                                      sel(inp["erase"]), sel(inp["write"]), s0, scheme=scheme, fg2=fg2,
                                      return_flags=True)
        o[0, :, h], S[0, h] = oo, SS
        flags += fl
    return o, S, flags


SCALAR_REGIMES = [("sigmoid", 3.0, 1.0), ("sigmoid", 1.0, 1.0), ("sigmoid", 0.0, 1.0), ("sigmoid", -1.0, 1.0)]
CHANNEL_REGIMES = [("softplus", -4.0, 1.5), ("softplus", -1.0, 1.5), ("softplus", 0.0, 1.5), ("softplus", 2.0, 1.5)]
CASES = ([("scalar",) + r for r in SCALAR_REGIMES] + [(v,) + r for v in ("kda", "decoupled", "fg2") for r in CHANNEL_REGIMES])


@pytest.mark.parametrize("variant,decay,mu,sd", CASES)
def test_safe_scheme_meets_bar_at_every_decay(variant, decay, mu, sd):
    inp = _inputs(variant, decay, mu, sd)
    ro, rS = _oracle(inp, variant == "fg2")
    o, S, _ = _emulate(inp, "safe", variant == "fg2")
    eo, eS = err_o(o, ro), err_S(S, rS)
    assert eo <= TOL_BF16 and eS <= TOL_BF16, (eo, eS)


@pytest.mark.parametrize("variant,decay,mu,sd", [("scalar", "sigmoid", 0.0, 1.0), ("kda", "softplus", -1.0, 1.5),
                                                 ("decoupled", "softplus", 0.0, 1.5)])
def test_midpoint_scheme_fails_under_strong_decay(variant, decay, mu, sd):
    # the planted mistake: the first kernel's referencing; it must fail the bar (or give NaN)
    inp = _inputs(variant, decay, mu, sd)
    ro, rS = _oracle(inp, False)
    with np.errstate(all="ignore"):
        o, S, _ = _emulate(inp, "midpoint", False)
    eo, eS = err_o(o, ro), err_S(S, rS)
    assert not (eo <= TOL_BF16 and eS <= TOL_BF16), (eo, eS)


def test_midpoint_scheme_passes_under_weak_decay():
    # ... and agrees with the safe scheme where its range holds (the regime every earlier test drew)
    inp = _inputs("kda", "softplus", -4.0, 1.5)
    ro, rS = _oracle(inp, False)
    o, S, _ = _emulate(inp, "midpoint", False)
    assert err_o(o, ro) <= TOL_BF16 and err_S(S, rS) <= TOL_BF16


def test_fast_and_level_paths_both_taken():
    # weak decay keeps every 16-token block on the midpoint split; strong decay moves them to the
    # level split; a wide spread mixes both within one chunk
    _, _, weak = _emulate(_inputs("kda", "softplus", -4.0, 1.5, T=256), "safe", False)
    _, _, strong = _emulate(_inputs("kda", "softplus", 2.0, 1.5, T=256), "safe", False)
    inp = _inputs("kda", "softplus", -4.0, 1.5, seed=5)
    hard = _inputs("kda", "softplus", 2.0, 1.5, seed=6)["log_decay"]
    inp["log_decay"][:, 64:96] = hard[:, 64:96]  # two strong blocks in the second chunk
    ro, rS = _oracle(inp, False)
    o, S, mixed = _emulate(inp, "safe", False)
    assert all(weak) and not any(strong)
    assert any(mixed) and not all(mixed)
    assert err_o(o, ro) <= TOL_BF16 and err_S(S, rS) <= TOL_BF16


@pytest.mark.parametrize("variant", ["scalar", "kda", "decoupled"])
def test_extreme_decay(variant):
    # log a down to about -60 per token (a ~ 1e-26): the state forgets within one token, and the
    # output is the current token's own write; the factors underflow only where they are negligible
    decay = "sigmoid" if variant == "scalar" else "softplus"
    mu = -40.0 if variant == "scalar" else 40.0
    inp = _inputs(variant, decay, mu, 10.0)
    ro, rS = _oracle(inp, False)
    o, S, _ = _emulate(inp, "safe", False)
    assert err_o(o, ro) <= TOL_BF16 and err_S(S, rS) <= TOL_BF16


@pytest.mark.parametrize("variant", ["scalar", "kda", "decoupled"])
@pytest.mark.parametrize("edge", ["no_decay", "no_erase", "full_gates"])
def test_edge_gates(variant, edge):
    # log a = 0; erase = 0 (with the symmetric gates the write vanishes too, with decoupled gates
    # this is gated linear attention); erase = write = 1 with unit keys (exact memory)
    import torch

    inp = _inputs(variant, "sigmoid" if variant == "scalar" else "softplus", 0.0, 1.5)
    if edge == "no_decay":
        inp["log_decay"] = torch.zeros_like(inp["log_decay"])
    elif edge == "no_erase":
        inp["erase"] = torch.zeros_like(inp["erase"])
    else:
        inp["erase"] = torch.ones_like(inp["erase"])
        if inp["write"] is not None:
            inp["write"] = torch.ones_like(inp["write"])
    ro, rS = _oracle(inp, False)
    o, S, _ = _emulate(inp, "safe", False)
    assert err_o(o, ro) <= TOL_BF16 and err_S(S, rS) <= TOL_BF16


def test_large_values():
    inp = _inputs("kda", "softplus", -1.0, 1.5, v_scale=1000.0)
    ro, rS = _oracle(inp, False)
    o, S, _ = _emulate(inp, "safe", False)
    assert err_o(o, ro) <= TOL_BF16 and err_S(S, rS) <= TOL_BF16


# ---- the gradients' chunk form --------------------------------------------------------------
# The matrix-core backward evaluates the gradients chunk by chunk from each chunk's incoming state
# and end adjoint (tests/chunk_model.py, ``chunk_backward``).  Its algebra must equal the adjoint
# of the token loop exactly (fp64, both the element-by-element and the kernels' block arrangement
# of the Gram adjoints, for every gate form and decay strength), and with fp16 operands where the
# kernels round it must stay inside the bf16 parity bar.
BWD_VARIANTS = ["scalar", "kda", "decoupled", "channel_shared", "fg2"]
BWD_REGIMES = [("softplus", -4.0, 1.5), ("sigmoid", 0.0, 1.5), ("softplus", 2.0, 1.0)]


def _bwd_case(variant, decay, mu, sd, T=150, d=32, seed=3):
    import torch

    from gated_delta_rule_dr_amd.workloads import Workload, generate

    wl = Workload("case", 1, T, 1, d, d, "f32", decay, variant != "scalar", mu, sd,
                  variant in ("decoupled", "channel_shared", "fg2"), "channel" if variant == "decoupled" else "erase",
                  0.05, seed, rate_sqrt=variant == "fg2")
    inp = generate(wl)
    g = torch.Generator().manual_seed(seed + 1)
    dO = torch.randn((1, T, 1, d), generator=g, dtype=torch.float64)
    dST = torch.randn((1, 1, d, d), generator=g, dtype=torch.float64)
    return inp, dO, dST


def _bwd_errors(variant, decay, mu, sd, blocked, fp16):
    from chunk_model import chunk_backward
    from oracle import recurrence_bwd, recurrence_fg2_bwd

    inp, dO, dST = _bwd_case(variant, decay, mu, sd)
    fg2 = variant == "fg2"
    if fg2:
        ref = recurrence_fg2_bwd(inp["q"], inp["k"], inp["v"], inp["log_decay"], inp["erase"], inp["S0"], dO, dST)
    else:
        ref = recurrence_bwd(inp["q"], inp["k"], inp["v"], inp["log_decay"], inp["erase"], inp["write"], inp["S0"],
                             dO=dO, dS_T=dST)
    sel = lambda x: None if x is None else _f(x)[0, :, 0]
    got = chunk_backward(sel(inp["q"]), sel(inp["k"]), sel(inp["v"]), sel(inp["log_decay"]), sel(inp["erase"]),
                         sel(inp["write"]), _f(inp["S0"])[0, 0], _f(dO)[0, :, 0], _f(dST)[0, 0], fg2=fg2,
                         blocked=blocked, fp16=fp16)
    errs = {}
    for key, x in got.items():
        if x is None:
            assert ref.get(key) is None
            continue
        r = ref[key][0, 0] if key == "dS0" else ref[key][0, :, 0]
        errs[key] = float(np.abs(x - r).max() / max(np.abs(r).max(), 1e-300))
    return errs


@pytest.mark.parametrize("variant", BWD_VARIANTS)
@pytest.mark.parametrize("decay,mu,sd", BWD_REGIMES)
def test_chunk_backward_algebra_exact(variant, decay, mu, sd):
    for blocked in (False, True):
        errs = _bwd_errors(variant, decay, mu, sd, blocked, False)
        assert max(errs.values()) <= 1e-12, (blocked, errs)


@pytest.mark.parametrize("variant", BWD_VARIANTS)
def test_chunk_backward_fp16_operands_meet_bar(variant):
    for decay, mu, sd in BWD_REGIMES:
        errs = _bwd_errors(variant, decay, mu, sd, True, True)
        assert max(errs.values()) <= TOL_BF16, (decay, mu, errs)

