"""The segment-parallel scan's algebra in fp64 (tests/chunk_model.py, segmented_forward): the
maps (F, H) of segments of whole chunks, chained S_in[s + 1] = F[s] S_in[s] + H[s], reproduce the
token recurrence of the oracle to rounding for every gate kind, for the library's segment plans
(tests/chunk_model.py, wide_plan) and for arbitrary ones; a dropped offset, a map taken in the
wrong order or a transposed map fails.  ("Linearized 2-Simplicial Attention" page, method;
"FG2-GDN" page, section 3.)"""
import numpy as np
import pytest

from chunk_model import segmented_forward, wide_plan
from metrics import err_S as _err_S
from metrics import err_o as _err_o
from oracle import recurrence


def err_o(o, ref):  # one (b, h): [T, dv]
    return _err_o(o[None, :, None], ref[None, :, None])


def err_S(S, ref):  # one (b, h): [dk, dv]
    return _err_S(S[None, None], ref[None, None])


def _one_head(variant, T, d, seed, s0=True, mu=-1.0, er_mu=0.0):
    g = np.random.default_rng(seed)
    q = g.standard_normal((T, d))
    k = g.standard_normal((T, d))
    k /= np.linalg.norm(k, axis=1, keepdims=True)
    v = g.standard_normal((T, d))
    la = -np.log1p(np.exp(g.normal(mu, 1.5, (T, d) if variant != "scalar" else (T,))))
    if variant == "decoupled":
        er = 1.0 / (1.0 + np.exp(-g.normal(er_mu, 1.0, (T, d))))
        wr = 1.0 / (1.0 + np.exp(-g.standard_normal((T, d))))
    elif variant == "head_write":
        er = 1.0 / (1.0 + np.exp(-g.standard_normal((T, d))))
        wr = 1.0 / (1.0 + np.exp(-g.standard_normal(T)))
    else:
        er = 1.0 / (1.0 + np.exp(-g.standard_normal(T)))
        wr = None
    S0 = 0.1 * g.standard_normal((d, d)) if s0 else None
    return q, k, v, la, er, wr, S0


def _oracle(q, k, v, la, er, wr, S0):
    x = [a[None, :, None] if a is not None else None for a in (q, k, v, la, er, wr)]
    ro, rS = recurrence(*x, None if S0 is None else S0[None, None])
    return ro[0, :, 0], rS[0, 0]


def _bounds(plan):
    P, L0, L = plan
    return [0] + [L0 + i * L for i in range(P - 1)]


@pytest.mark.parametrize("mu", [-1.0, -6.0])  # strong decay (segments forget) and weak (F matters)
@pytest.mark.parametrize("variant", ["decoupled", "head_write", "kda", "scalar"])
@pytest.mark.parametrize("bh,T", [(32, 64 * 20), (2, 64 * 9 + 7), (1, 64 * 5 + 33), (1, 130)])
def test_library_plans_match_oracle(variant, bh, T, mu):
    P, L0, L = wide_plan(bh, T)
    nch = -(-T // 64)
    assert P >= 1 and L0 >= 1 and (P == 1 or (L >= 1 and L0 + (P - 1) * L == nch))
    inp = _one_head(variant, T, 32, seed=T + bh, mu=mu)
    o, S, Fs, Hs = segmented_forward(*inp, bounds=_bounds((P, L0, L)))
    ro, rS = _oracle(*inp)
    assert len(Fs) == P - 1
    assert err_o(o, ro) < 1e-11 and err_S(S, rS) < 1e-11, (err_o(o, ro), err_S(S, rS))


@pytest.mark.parametrize("bounds", [[0, 1], [0, 3, 4, 9], [0, 2, 4, 6, 8, 10, 12, 14, 16, 18]])
def test_arbitrary_segments_match_oracle(bounds):
    inp = _one_head("decoupled", 64 * 20, 32, seed=len(bounds), mu=-6.0)
    o, S, _, _ = segmented_forward(*inp, bounds=bounds)
    ro, rS = _oracle(*inp)
    assert err_o(o, ro) < 1e-11 and err_S(S, rS) < 1e-11


def test_plan_shapes():
    # every shape the plan takes: one segment, two, a first segment longer than the others, and
    # the bench shape (32 heads of 1,024 chunks: nine segments, the first of 88 chunks)
    assert wide_plan(2, 130) == (1, 3, 3)
    assert wide_plan(1, 300) == (2, 3, 2)
    assert wide_plan(2, 520) == (4, 3, 2)
    assert wide_plan(32, 65536) == (9, 88, 117)
    assert wide_plan(256, 65536)[0] == 1


@pytest.mark.parametrize("mistake", ["no_offset", "reversed", "transposed"])
def test_planted_mistakes_fail(mistake):
    # the composition done wrong, on the same maps, must miss the oracle by far (one-chunk
    # segments with weak decay and weak erasure, so that a segment's map F carries its entering
    # state: |F| is not small)
    q, k, v, la, er, wr, S0 = _one_head("decoupled", 64 * 4, 32, seed=5, mu=-7.0, er_mu=-4.0)
    bounds = [0, 1, 2, 3]
    _, _, Fs, Hs = segmented_forward(q, k, v, la, er, wr, S0, bounds=bounds)
    assert min(np.abs(F).max() for F in Fs) > 0.5
    S = S0.copy()
    for F, Hm in zip(Fs, Hs):
        if mistake == "no_offset":
            S = F @ S
        elif mistake == "reversed":
            S = S @ F + Hm
        else:
            S = F.T @ S + Hm
    # the state entering the last segment, from the oracle's state after token 3 * 64
    _, rS = _oracle(q[:192], k[:192], v[:192], la[:192], er[:192], wr[:192], S0)
    assert err_S(S, rS) > 1e-3
    # and done right it matches
    S = S0.copy()
    for F, Hm in zip(Fs, Hs):
        S = F @ S + Hm
    assert err_S(S, rS) < 1e-11
