"""GPU parity at the workloads' full sizes, in the launch configuration bench.py times.

Each prefill workload runs once at full size on the device (inputs drawn with the device
generator); the fp64 oracle then recomputes a few sampled (b, h) pairs -- first, last and one
inside -- from the very same input values, over the whole sequence, and o and S_T of those
pairs must agree to the bf16-path tolerance; every head is checked for finiteness.  The decode
workload runs its full 256 x 32 heads for a number of steps and samples (n, h) pairs the same
way, and one sequence (all its heads) follows the oracle over all 1,000 steps of the workload;
the packed serving workload samples (sequence, head) pairs.  A linearity identity covers every
head of a prefill workload."""
import pytest
import torch

from metrics import err_S, err_o
from oracle import decode_step as oracle_decode
from oracle import recurrence, recurrence_fg2

pytestmark = pytest.mark.gpu

TOL_BF16 = 3e-3
TOL_F32 = 1e-5


@pytest.fixture(scope="module")
def dr():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gated_delta_rule_dr_amd as m

    m.abi_version()
    return m


def _slice(x, b, h):
    """Inputs of one (b, h) as a [1, T, 1, ...] CPU tensor."""
    if x is None:
        return None
    return x[b:b + 1, :, h:h + 1].cpu()


@pytest.mark.parametrize("name,pairs", [
    ("gdn_scalar_bf16_t4k", [(0, 0), (1, 7), (3, 15)]),
    ("kda_channel_bf16_t16k", [(0, 0), (1, 31)]),
    ("fg2_channel_bf16_t16k", [(0, 0), (1, 31)]),
    ("gdn2_decoupled_bf16_t64k", [(0, 0), (0, 31)]),
])
def test_prefill_full_size_sampled_heads(dr, name, pairs):
    from gated_delta_rule_dr_amd.workloads import generate, workload

    wl = workload(name)
    inp = generate(wl, device="cuda")
    o = torch.empty((wl.B, wl.T, wl.H, wl.dv), device="cuda")
    S_T = torch.empty((wl.B, wl.H, wl.dk, wl.dv), device="cuda")
    dr.chunk_fwd(inp["q"], inp["k"], inp["v"], inp["log_decay"], inp["erase"], inp["write"], inp["S0"],
                 out=o, S_T=S_T, fg2=wl.rate_sqrt)
    torch.cuda.synchronize()
    assert torch.isfinite(o).all() and torch.isfinite(S_T).all()
    print(f"{name}: |o|max={o.abs().max().item():.3g} |S_T|max={S_T.abs().max().item():.3g}", flush=True)
    for b, h in pairs:
        sl = {k: _slice(v, b, h) for k, v in inp.items()}
        if wl.rate_sqrt:
            ro, rS = recurrence_fg2(sl["q"], sl["k"], sl["v"], sl["log_decay"], sl["erase"], sl["S0"])
        else:
            ro, rS = recurrence(sl["q"], sl["k"], sl["v"], sl["log_decay"], sl["erase"], sl["write"], sl["S0"])
        eo = err_o(o[b:b + 1, :, h:h + 1], ro)
        eS = err_S(S_T[b:b + 1, h:h + 1], rS)
        print(f"{name} (b={b}, h={h}): err_o={eo:.3e} err_S={eS:.3e}", flush=True)
        assert eo <= TOL_BF16 and eS <= TOL_BF16, (b, h, eo, eS)


def test_packed_full_size_sampled_sequences(dr):
    """The packed serving workload at full size, as bench.py times it: sampled (sequence, head)
    pairs -- the first sequence, the longest and the last -- against the oracle over each
    whole sequence."""
    from gated_delta_rule_dr_amd.workloads import generate, seq_lengths, workload

    wl = workload("gdn_scalar_bf16_varlen_t16k")
    inp = generate(wl, device="cuda")
    lens = seq_lengths(wl)
    N = len(lens)
    o = torch.empty((1, wl.T, wl.H, wl.dv), device="cuda")
    S_T = torch.empty((N, wl.H, wl.dk, wl.dv), device="cuda")
    dr.chunk_fwd_varlen(inp["q"], inp["k"], inp["v"], inp["log_decay"], inp["erase"], inp["write"], inp["S0"],
                        cu_seqlens=inp["cu_seqlens"], out=o, S_T=S_T)
    torch.cuda.synchronize()
    assert torch.isfinite(o).all() and torch.isfinite(S_T).all()
    cu = inp["cu_seqlens"].cpu().tolist()
    longest = max(range(N), key=lambda n: lens[n])
    for n, h in [(0, 0), (longest, 7), (N - 1, wl.H - 1)]:
        lo, hi = cu[n], cu[n + 1]
        sl = {k: (None if v is None else v[:, lo:hi, h:h + 1].cpu())
              for k, v in inp.items() if k not in ("cu_seqlens", "S0")}
        ro, rS = recurrence(sl["q"], sl["k"], sl["v"], sl["log_decay"], sl["erase"], sl["write"], None)
        eo = err_o(o[:, lo:hi, h:h + 1], ro)
        eS = err_S(S_T[n:n + 1, h:h + 1], rS)
        print(f"packed (sequence {n} of {hi - lo} tokens, h={h}): err_o={eo:.3e} err_S={eS:.3e}", flush=True)
        assert eo <= TOL_BF16 and eS <= TOL_BF16, (n, h, eo, eS)


def test_prefill_full_size_linearity_all_heads(dr):
    """With the gates fixed, (S0, V) -> (O, S_T) is linear, so o(2v) = 2 o(v) and S_T likewise
    on every head of the full bench workload.  The chunk path meets this only to its rounding
    level: fp16 operands that fall in the subnormal range round on a fixed absolute grid, so
    doubling them does not double their rounding (the matrix cores and normal-range
    conversions do scale exactly); the resulting one-ulp differences can flip the fp16
    rounding of a state operand in a later chunk, which moves that chunk by one fp16 step
    (measured: 1e-4 normwise), so the bound is the bf16-path tolerance."""
    from gated_delta_rule_dr_amd.workloads import generate, workload

    wl = workload("gdn_scalar_bf16_t4k")
    inp = generate(wl, device="cuda")
    o1, S1 = dr.chunk_fwd(inp["q"], inp["k"], inp["v"], inp["log_decay"], inp["erase"], None, None)
    o2, S2 = dr.chunk_fwd(inp["q"], inp["k"], inp["v"] * 2, inp["log_decay"], inp["erase"], None, None)
    torch.cuda.synchronize()
    eo, eS = err_o(o2 / 2, o1), err_S(S2 / 2, S1)
    print(f"linearity: err_o={eo:.3e} err_S={eS:.3e}", flush=True)
    assert eo <= TOL_BF16 and eS <= TOL_BF16


def test_decode_all_steps_one_sequence(dr):
    # the decode workload's full length: all 1,000 steps on all 256 x 32 heads, as bench.py runs
    # them; sequence 137 (all 32 heads) follows the oracle's token steps from the same inputs, o
    # at every step and S after the last
    from gated_delta_rule_dr_amd.workloads import generate_decode, workload

    wl = workload("decode_kda_n256_h32")
    n = 137
    inp = generate_decode(wl, steps=wl.steps, device="cuda")
    S = inp["S0"].clone()
    o = torch.empty((wl.B, wl.H, wl.dv), device="cuda")
    o_seq = torch.empty((wl.steps, wl.H, wl.dv), device="cuda")
    for s in range(wl.steps):
        g = lambda key: None if inp[key] is None else inp[key][s]
        dr.decode_step(g("q"), g("k"), g("v"), g("log_decay"), g("erase"), g("write"), S=S, o=o)
        o_seq[s].copy_(o[n])
    torch.cuda.synchronize()
    cut = lambda key: None if inp[key] is None else inp[key][:, n:n + 1].cpu()
    seq = {key: cut(key) for key in ("q", "k", "v", "log_decay", "erase", "write")}
    refS = inp["S0"][n:n + 1].double().cpu().numpy()
    del inp
    worst = 0.0
    o_seq = o_seq.cpu()
    for s in range(wl.steps):
        g = lambda key: None if seq[key] is None else seq[key][s]
        ro, refS = oracle_decode(g("q"), g("k"), g("v"), g("log_decay"), g("erase"), g("write"), refS)
        worst = max(worst, err_o(o_seq[s][None, None], ro[:, None]))
    eS = err_S(S[n:n + 1], refS)
    print(f"decode sequence {n}, {wl.H} heads, {wl.steps} steps: max err_o={worst:.3e} err_S={eS:.3e}", flush=True)
    assert worst <= TOL_F32 and eS <= TOL_F32
    assert torch.isfinite(S).all()


def test_decode_full_size_sampled_pairs(dr):
    from gated_delta_rule_dr_amd.workloads import generate_decode, workload

    wl = workload("decode_kda_n256_h32")
    steps = 16
    inp = generate_decode(wl, steps=steps, device="cuda")
    pairs = [(0, 0), (100, 17), (255, 31)]
    S = inp["S0"].clone()
    refS = {pr: inp["S0"][pr[0]:pr[0] + 1, pr[1]:pr[1] + 1].double().cpu().numpy() for pr in pairs}
    o = torch.empty((wl.B, wl.H, wl.dv), device="cuda")
    for s in range(steps):
        g = lambda key: None if inp[key] is None else inp[key][s]
        dr.decode_step(g("q"), g("k"), g("v"), g("log_decay"), g("erase"), g("write"), S=S, o=o)
        torch.cuda.synchronize()
        for n, h in pairs:
            cut = lambda x: None if x is None else x[n:n + 1, h:h + 1].cpu()
            ro, refS[(n, h)] = oracle_decode(cut(g("q")), cut(g("k")), cut(g("v")), cut(g("log_decay")),
                                             cut(g("erase")), cut(g("write")), refS[(n, h)])
            eo = err_o(o[n:n + 1, h:h + 1][:, None], ro[:, None])
            assert eo <= TOL_F32, (s, n, h, eo)
    for n, h in pairs:
        eS = err_S(S[n:n + 1, h:h + 1], refS[(n, h)])
        print(f"decode (n={n}, h={h}) after {steps} steps: err_S={eS:.3e}", flush=True)
        assert eS <= TOL_F32
    assert torch.isfinite(S).all()
