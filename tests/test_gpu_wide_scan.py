"""GPU parity of the full-width segmented scan (separate erase and write gates over a dense batch).

The scan cuts each sequence into P segments by a plan that depends on B * H and the chunk count:
P - 1 = min(256 / (B * H), 8), at most half the chunks, segment 0 about 0.7 times as long as the
others.  The cases below are chosen so that the plan takes each of its shapes: one segment (no
maps, no composition), two (no composition step), three and four (short segments, segment 0
longer than the others), and nine (the bench shape's count), with ragged last chunks, an initial
state, a per-channel or a per-head write gate, and bf16 output.  Each is checked against the fp64
oracle ("Gated DeltaNet-2" page, the solution and its gate table; "FG2-GDN" page, section 2, the
update rule) at the 3e-3 bar of the bf16 matrix-core path.
"""
import numpy as np
import pytest
import torch

from chunk_model import wide_plan
from metrics import err_S, err_o
from oracle import recurrence

pytestmark = pytest.mark.gpu

TOL_BF16 = 3e-3
TOL_BF16_O = TOL_BF16 + 2 ** -8  # bf16 o: the path's bar plus the output format's own rounding


@pytest.fixture(scope="module")
def dr():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gated_delta_rule_dr_amd as m

    m.abi_version()
    return m


def _inputs(B, T, H, write_per_channel, s0, seed):
    from gated_delta_rule_dr_amd.workloads import Workload, generate

    wl = Workload("case", B, T, H, 128, 128, "bf16", "softplus", True, -2.0, 1.5, True, "channel",
                  0.05 if s0 else 0.0, seed)
    inp = generate(wl)
    if not write_per_channel:
        # one write gate per (b, t, h) beside the per-channel erase gate
        g = np.random.default_rng(seed + 7)
        inp["write"] = torch.from_numpy(1.0 / (1.0 + np.exp(-g.standard_normal((B, T, H))))).float()
    return inp


# (B, T, H, expected segments)
SHAPES = [(1, 130, 2, 1), (1, 300, 1, 2), (1, 64 * 6 + 10, 1, 3), (2, 520, 1, 4), (1, 1280, 32, 9)]


@pytest.mark.parametrize("B,T,H,P", SHAPES)
@pytest.mark.parametrize("write_per_channel", [True, False])
def test_wide_scan_segment_plans(dr, B, T, H, P, write_per_channel):
    assert wide_plan(B * H, T)[0] == P
    inp = _inputs(B, T, H, write_per_channel, s0=True, seed=T + H + int(write_per_channel))
    d = {k: (None if v is None else v.cuda()) for k, v in inp.items()}
    o, S = dr.chunk_fwd(d["q"], d["k"], d["v"], d["log_decay"], d["erase"], d["write"], d["S0"])
    torch.cuda.synchronize()
    ro, rS = recurrence(inp["q"], inp["k"], inp["v"], inp["log_decay"], inp["erase"], inp["write"], inp["S0"])
    eo, eS = err_o(o, ro), err_S(S, rS)
    print(f"B={B} T={T} H={H} P={P} write_per_channel={write_per_channel}: err_o={eo:.2e} err_S={eS:.2e}")
    assert eo <= TOL_BF16 and eS <= TOL_BF16, (eo, eS)


def test_wide_scan_bf16_output_and_state_in_place(dr):
    # nine segments, bf16 o, and S_T written over S0 (the first phase reads S0 before the second
    # phase writes S_T)
    B, T, H = 1, 1280, 32
    inp = _inputs(B, T, H, True, s0=True, seed=77)
    d = {k: (None if v is None else v.cuda()) for k, v in inp.items()}
    S = d["S0"].clone()
    o, S_out = dr.chunk_fwd(d["q"], d["k"], d["v"], d["log_decay"], d["erase"], d["write"], S, S_T=S,
                            o_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    ro, rS = recurrence(inp["q"], inp["k"], inp["v"], inp["log_decay"], inp["erase"], inp["write"], inp["S0"])
    eo, eS = err_o(o.float(), ro), err_S(S, rS)
    print(f"bf16 o, in place: err_o={eo:.2e} err_S={eS:.2e}")
    assert eo <= TOL_BF16_O and eS <= TOL_BF16, (eo, eS)
    assert S_out.data_ptr() == S.data_ptr()


def test_wide_scan_deterministic(dr):
    B, T, H = 1, 1280, 32
    inp = _inputs(B, T, H, True, s0=True, seed=78)
    d = {k: (None if v is None else v.cuda()) for k, v in inp.items()}
    outs = [dr.chunk_fwd(d["q"], d["k"], d["v"], d["log_decay"], d["erase"], d["write"], d["S0"]) for _ in range(2)]
    torch.cuda.synchronize()
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])
