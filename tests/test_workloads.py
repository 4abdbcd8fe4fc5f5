"""Seeded input generators: shapes, dtypes, value ranges and determinism (CPU only)."""
import torch

from gated_delta_rule_dr_amd.workloads import WORKLOADS, generate, generate_decode, seq_lengths, workload


def test_shapes_dtypes_and_ranges_small():
    for name, wl in WORKLOADS.items():
        if wl.steps:
            small = wl.replace(B=3, H=2)
            d = generate_decode(small, steps=4)
            assert d["q"].shape == (4, 3, 2, 128) and d["q"].dtype == torch.bfloat16
            assert d["S0"].shape == (3, 2, 128, 128) and d["S0"].dtype == torch.float32
            assert d["log_decay"].shape == (4, 3, 2, 128)
            assert d["erase"].shape == (4, 3, 2)
            assert abs(float(d["S0"].std()) - 0.01) < 1e-3
            continue
        small = wl.replace(B=1, T=70, H=2)
        d = generate(small)
        dt = torch.bfloat16 if wl.qkv_dtype == "bf16" else torch.float32
        assert d["q"].dtype == dt and d["k"].dtype == dt and d["v"].dtype == dt
        assert d["q"].shape == (1, 70, 2, wl.dk) and d["v"].shape == (1, 70, 2, wl.dv)
        ld = d["log_decay"]
        assert ld.dtype == torch.float32 and bool((ld <= 0).all())
        assert ld.shape == ((1, 70, 2, wl.dk) if wl.decay_channel else (1, 70, 2))
        assert bool(((d["erase"] > 0) & (d["erase"] < 1)).all())
        assert (d["write"] is None) == (wl.write == "erase")
        norms = torch.linalg.vector_norm(d["k"].double(), dim=-1)
        assert float((norms - 1).abs().max()) < 1e-2  # unit keys up to the storage rounding
        assert d["S0"] is None
        assert ("cu_seqlens" in d) == (wl.seq_median > 0)


def test_seeded_and_deterministic():
    wl = workload("kda_channel_bf16_t16k", B=1, T=33, H=2)
    a, b = generate(wl), generate(wl)
    for key in ("q", "k", "v", "log_decay", "erase"):
        assert torch.equal(a[key], b[key])
    c = generate(wl.replace(seed=99))
    assert not torch.equal(a["q"], c["q"])


def test_decay_distribution_matches_recipe():
    # log alpha = log sigmoid(N(3,1)): alpha has mean about 0.93
    wl = workload("gdn_scalar_f32_d32", T=4096, H=8)
    alpha = torch.exp(generate(wl)["log_decay"].double())
    assert 0.90 < float(alpha.mean()) < 0.95


def test_packed_lengths_recipe():
    wl = workload("gdn_scalar_bf16_varlen_t16k")
    lens = seq_lengths(wl)
    assert sum(lens) == wl.T and min(lens) >= 1 and max(lens) <= wl.seq_max
    assert lens == seq_lengths(wl)  # seeded
    assert 10 <= len(lens) <= 200
    small = wl.replace(T=3000, H=2, s0_std=0.1)
    d = generate(small)
    cu = d["cu_seqlens"]
    assert cu.dtype == torch.int32 and int(cu[0]) == 0 and int(cu[-1]) == 3000
    assert bool((cu[1:] >= cu[:-1]).all())
    assert d["q"].shape == (1, 3000, 2, 128)
    assert d["S0"].shape == (cu.numel() - 1, 2, 128, 128)
