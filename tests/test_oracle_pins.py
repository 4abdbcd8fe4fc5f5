"""Pins for the fp64 oracle: checks against facts fixed by the pages and by mathematics, each
chosen so that a plausible slip in the oracle (a dropped term, a wrong sign or index, decay
applied after the erase, reading the state before the write, a transposed operand) fails at
least one of them.  CPU only."""
import json
import os

import numpy as np
import pytest

from chunk_model import chunk_forward
from oracle import decode_step, recurrence, recurrence_bwd, recurrence_fg2, recurrence_fg2_bwd, recurrence_varlen

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


def _unit(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def _sig(x):
    return 1.0 / (1.0 + np.exp(-x))


def _inputs(seed, B=2, T=23, H=3, dk=5, dv=4, decay="channel", erase="channel", write="channel",
            s0=True, unit_k=True):
    r = _rng(seed)
    q = r.standard_normal((B, T, H, dk))
    k = r.standard_normal((B, T, H, dk))
    if unit_k:
        k = _unit(k)
    v = r.standard_normal((B, T, H, dv))
    ld = -np.log1p(np.exp(r.normal(-2.0, 1.0, (B, T, H) + ((dk,) if decay == "channel" else ()))))
    e = _sig(r.standard_normal((B, T, H) + ((dk,) if erase == "channel" else ())))
    w = None
    if write == "channel":
        w = _sig(r.standard_normal((B, T, H, dv)))
    elif write == "head":
        w = _sig(r.standard_normal((B, T, H)))
    S0 = r.standard_normal((B, H, dk, dv)) if s0 else None
    return q, k, v, ld, e, w, S0


# P1 -- erase = 0, decay = 1, write = 1 reduces to causal linear attention with a fixed-size
# state ("KronLSTM ...", The problem; "Gated DeltaNet-2 ...", the attention bottleneck):
# o_t = S0^T q_t + sum_{j<=t} (q_t . k_j) v_j, computed here by brute force over token pairs.
def test_linear_attention_bruteforce():
    q, k, v, _, _, _, S0 = _inputs(1, unit_k=False)
    B, T, H, dk = q.shape
    zeros = np.zeros((B, T, H))
    o, S = recurrence(q, k, v, zeros, zeros, np.ones((B, T, H)), S0)
    ref = np.zeros_like(o)
    for b in range(B):
        for h in range(H):
            for t in range(T):
                acc = S0[b, h].T @ q[b, t, h]
                for j in range(t + 1):
                    acc = acc + np.dot(q[b, t, h], k[b, j, h]) * v[b, j, h]
                ref[b, t, h] = acc
    assert np.max(np.abs(o - ref)) <= 1e-12 * np.max(np.abs(ref))
    S_ref = S0 + np.einsum("bthi,bthj->bhij", k, v)
    assert np.allclose(S, S_ref, rtol=0, atol=1e-12)


# P2 -- erase = 0 leaves gated linear attention, whose closed form uses the global cumulative
# log-decay G_t = sum_{i<=t} log a_i:
#   o_t = (q_t e^{G_t})^T S0 + sum_{j<=t} ((q_t e^{G_t - G_j}) . k_j) (w_j v_j)
@pytest.mark.parametrize("decay", ["channel", "head"])
def test_gated_linear_attention_closed_form(decay):
    q, k, v, ld, _, w, S0 = _inputs(2, decay=decay, T=17)
    B, T, H, dk = q.shape
    zeros = np.zeros((B, T, H))
    o, S = recurrence(q, k, v, ld, zeros, w, S0)
    ldc = ld if ld.ndim == 4 else np.broadcast_to(ld[..., None], q.shape)
    G = np.cumsum(ldc, axis=1)
    ref = np.zeros_like(o)
    S_ref = np.zeros_like(S)
    for b in range(B):
        for h in range(H):
            for t in range(T):
                acc = (q[b, t, h] * np.exp(G[b, t, h])) @ S0[b, h]
                for j in range(t + 1):
                    coef = np.dot(q[b, t, h] * np.exp(G[b, t, h] - G[b, j, h]), k[b, j, h])
                    acc = acc + coef * (w[b, j, h] * v[b, j, h])
                ref[b, t, h] = acc
            Sr = np.exp(G[b, T - 1, h])[:, None] * S0[b, h]
            for j in range(T):
                Sr = Sr + np.outer(k[b, j, h] * np.exp(G[b, T - 1, h] - G[b, j, h]), w[b, j, h] * v[b, j, h])
            S_ref[b, h] = Sr
    assert np.max(np.abs(o - ref)) <= 1e-12 * np.max(np.abs(ref))
    assert np.max(np.abs(S - S_ref)) <= 1e-12 * np.max(np.abs(S_ref))


# P3 -- full erase and write with unit keys and no decay make each step a Householder
# projection followed by a write, so the memory returns exactly the value just stored:
# S_t^T k_t = v_t ("FG2-GDN", section 2: rank-1 Householder structure of the update).
def test_exact_memory_unit_keys():
    q, k, v, _, _, _, S0 = _inputs(3, T=31, dk=6, dv=6)
    B, T, H, _ = q.shape
    ones, zeros = np.ones((B, T, H)), np.zeros((B, T, H))
    _, _, states = recurrence(q, k, v, zeros, ones, None, S0, return_states=True)
    for t in range(T):
        readback = np.einsum("bhij,bhi->bhj", states[:, :, t], k[:, t])
        assert np.max(np.abs(readback - v[:, t])) <= 1e-12


# P4 -- per-step key readback identity for every variant (general form):
#   S_t^T k_t = (1 - k_t . u_t) S'^T k_t + ||k_t||^2 (w_t v_t),  S' = Diag(a_t) S_{t-1}
@pytest.mark.parametrize("variant", ["scalar", "kda", "decoupled"])
def test_key_readback_identity(variant):
    if variant == "scalar":
        args = dict(decay="head", erase="head", write=None)
    elif variant == "kda":
        args = dict(decay="channel", erase="head", write=None)
    else:
        args = dict(decay="channel", erase="channel", write="channel")
    q, k, v, ld, e, w, S0 = _inputs(4, unit_k=False, dk=4, dv=4, **args)
    B, T, H, dk = q.shape
    _, _, states = recurrence(q, k, v, ld, e, w, S0, return_states=True)
    a = np.exp(ld if ld.ndim == 4 else ld[..., None] * np.ones(dk))
    ee = e if e.ndim == 4 else e[..., None] * np.ones(dk)
    ww = (e if w is None else w)
    ww = ww if ww.ndim == 4 else ww[..., None] * np.ones(v.shape[-1])
    prev = S0
    for t in range(T):
        Sp = a[:, t][..., :, None] * prev
        m = np.einsum("bhij,bhi->bhj", Sp, k[:, t])
        ku = np.sum(k[:, t] * ee[:, t] * k[:, t], axis=-1)
        kk = np.sum(k[:, t] ** 2, axis=-1)
        expect = (1 - ku)[..., None] * m + kk[..., None] * ww[:, t] * v[:, t]
        got = np.einsum("bhij,bhi->bhj", states[:, :, t], k[:, t])
        assert np.max(np.abs(got - expect)) <= 1e-11 * max(1.0, np.max(np.abs(expect)))
        prev = states[:, :, t]


# P5 -- hand-worked 2x2 example (tests/golden, derivation in the fixture).
def test_worked_example_2x2():
    with open(os.path.join(GOLDEN, "worked_example_scalar_gdn_2x2.json")) as f:
        ex = json.load(f)
    toks = ex["tokens"]
    T = len(toks)
    arr = lambda key: np.array([tk[key] for tk in toks], np.float64)
    q, k, v = arr("q")[None, :, None], arr("k")[None, :, None], arr("v")[None, :, None]
    la = np.log(arr("alpha"))[None, :, None]
    beta = arr("beta")[None, :, None]
    o, S, states = recurrence(q, k, v, la, beta, None, None, return_states=True)
    for t in range(T):
        assert np.allclose(states[0, 0, t], np.array(toks[t]["S"]), rtol=0, atol=1e-14)
        assert np.allclose(o[0, t, 0], np.array(toks[t]["o"]), rtol=0, atol=1e-14)


def _explicit_loop(step, q, k, v, S0, T):
    S, o = S0.copy(), []
    for t in range(T):
        S = step(t, S)
        o.append(S.T @ q[t])
    return np.array(o), S


# P6 -- the explicit matrix forms each page states, written as products of dense matrices:
#   scalar GDN: S_t = alpha_t (I - beta_t k k^T) S_{t-1} + beta_t k v^T
#   KDA:        S_t = (I - beta_t k k^T) Diag(a_t) S_{t-1} + beta_t k v^T  ("FG2-GDN" section 1-2)
#   FG2-GDN:    kt = sqrt(beta) k, vt = sqrt(beta) v, S_t = (I - kt kt^T) Diag(a_t) S + kt vt^T
#               (per-channel beta; fed to the oracle as pre-scaled k, v with erase = write = 1)
#   GDN-2 / FG2-GDN+: S_t = (I - (b k) k^T) Diag(a_t) S + k (w v)^T  (erase on the key side,
#               write on the value side, "Gated DeltaNet-2 ...", gate table)
@pytest.mark.parametrize("form", ["scalar", "kda", "fg2", "decoupled"])
def test_explicit_matrix_forms(form):
    r = _rng(6)
    T, d = 19, 5
    q, v = r.standard_normal((T, d)), r.standard_normal((T, d))
    k = _unit(r.standard_normal((T, d)))
    S0 = r.standard_normal((d, d))
    a_vec = np.exp(-np.log1p(np.exp(r.normal(-2, 1, (T, d)))))
    alpha = np.exp(-np.log1p(np.exp(r.normal(-2, 1, T))))
    beta = _sig(r.standard_normal(T))
    bvec, wvec = _sig(r.standard_normal((T, d))), _sig(r.standard_normal((T, d)))
    I = np.eye(d)
    wrap = lambda x: x[None, :, None]
    if form == "scalar":
        step = lambda t, S: alpha[t] * (I - beta[t] * np.outer(k[t], k[t])) @ S + beta[t] * np.outer(k[t], v[t])
        o, S = recurrence(wrap(q), wrap(k), wrap(v), wrap(np.log(alpha)), wrap(beta), None, S0[None, None])
    elif form == "kda":
        step = lambda t, S: (I - beta[t] * np.outer(k[t], k[t])) @ np.diag(a_vec[t]) @ S + beta[t] * np.outer(k[t], v[t])
        o, S = recurrence(wrap(q), wrap(k), wrap(v), wrap(np.log(a_vec)), wrap(beta), None, S0[None, None])
    elif form == "fg2":
        kt, vt = np.sqrt(bvec) * k, np.sqrt(bvec) * v
        step = lambda t, S: (I - np.outer(kt[t], kt[t])) @ np.diag(a_vec[t]) @ S + np.outer(kt[t], vt[t])
        ones = np.ones(T)
        o, S = recurrence(wrap(q), wrap(kt), wrap(vt), wrap(np.log(a_vec)), wrap(ones), None, S0[None, None])
    else:
        step = lambda t, S: (I - np.outer(bvec[t] * k[t], k[t])) @ np.diag(a_vec[t]) @ S + np.outer(k[t], wvec[t] * v[t])
        o, S = recurrence(wrap(q), wrap(k), wrap(v), wrap(np.log(a_vec)), wrap(bvec), wrap(wvec), S0[None, None])
    o_ref, S_ref = _explicit_loop(step, q, k, v, S0, T)
    assert np.max(np.abs(o[0, :, 0] - o_ref)) <= 1e-12 * np.max(np.abs(o_ref))
    assert np.max(np.abs(S[0, 0] - S_ref)) <= 1e-12 * np.max(np.abs(S_ref))


# P6b -- variant plumbing: decoupled gates with b = w = beta*1 equal KDA; KDA with a = alpha*1
# equals the scalar-decay form.
def test_variant_reductions():
    q, k, v, ld, e, _, S0 = _inputs(7, decay="channel", erase="head", write=None)
    dk = q.shape[-1]
    o1, S1 = recurrence(q, k, v, ld, e, None, S0)
    ech = np.broadcast_to(e[..., None], e.shape + (dk,))
    o2, S2 = recurrence(q, k, v, ld, ech, ech[..., : v.shape[-1]] if v.shape[-1] <= dk else None, S0)
    assert np.allclose(o1, o2, rtol=0, atol=1e-13) and np.allclose(S1, S2, rtol=0, atol=1e-13)
    ld_head = ld[..., 0]
    o3, S3 = recurrence(q, k, v, ld_head, e, None, S0)
    o4, S4 = recurrence(q, k, v, np.broadcast_to(ld_head[..., None], ld.shape), e, None, S0)
    assert np.allclose(o3, o4, rtol=0, atol=1e-13) and np.allclose(S3, S4, rtol=0, atol=1e-13)


# P6c -- the online-learning reading of the delta rule ("FG2-GDN", section 2, the update as a
# gradient step with a (diagonal) learning rate): without decay, one step with scalar beta is
# S_t = S_{t-1} - beta grad L(S_{t-1}),  L(S) = 1/2 ||S^T k - v||^2, the gradient taken here by
# central finite differences (exact for a quadratic up to rounding).
def test_delta_rule_is_gradient_step():
    r = _rng(8)
    dk, dv = 4, 3
    S = r.standard_normal((dk, dv))
    k, v, q = _unit(r.standard_normal(dk)), r.standard_normal(dv), r.standard_normal(dk)
    beta = 0.37
    L = lambda X: 0.5 * np.sum((X.T @ k - v) ** 2)
    grad = np.zeros_like(S)
    h = 1e-3
    for i in range(dk):
        for j in range(dv):
            E = np.zeros_like(S)
            E[i, j] = h
            grad[i, j] = (L(S + E) - L(S - E)) / (2 * h)
    expect = S - beta * grad
    o, S1 = recurrence(q[None, None, None], k[None, None, None], v[None, None, None],
                       np.zeros((1, 1, 1)), np.full((1, 1, 1), beta), None, S[None, None])
    assert np.max(np.abs(S1[0, 0] - expect)) <= 1e-9
    assert np.max(np.abs(o[0, 0, 0] - expect.T @ q)) <= 1e-9


# P7 -- with the gates fixed, (S0, V) -> (O, S_T) is linear.
def test_linearity_in_state_and_values():
    q, k, v, ld, e, w, S0 = _inputs(9)
    _, _, v2, _, _, _, S02 = _inputs(10)
    o1, S1 = recurrence(q, k, v, ld, e, w, S0)
    o2, S2 = recurrence(q, k, v2, ld, e, w, S02)
    o3, S3 = recurrence(q, k, 2.0 * v + v2, ld, e, w, 2.0 * S0 + S02)
    assert np.allclose(o3, 2 * o1 + o2, rtol=0, atol=1e-12)
    assert np.allclose(S3, 2 * S1 + S2, rtol=0, atol=1e-12)
    o4, S4 = recurrence(q, k, 2.0 * v, ld, e, w, 2.0 * S0)
    assert np.array_equal(o4, 2 * o1) and np.array_equal(S4, 2 * S1)


# P9 -- the state is the checkpoint: running T tokens equals running T1 tokens and resuming
# from their final state for the remaining ones (bit-identical in fp64).
@pytest.mark.parametrize("split", [1, 11, 22])
def test_resume_from_state(split):
    q, k, v, ld, e, w, S0 = _inputs(11)
    o, S = recurrence(q, k, v, ld, e, w, S0)
    cut = lambda x: (x[:, :split], x[:, split:])
    oa, Sa = recurrence(*(cut(x)[0] for x in (q, k, v, ld, e, w)), S0)
    ob, Sb = recurrence(*(cut(x)[1] for x in (q, k, v, ld, e, w)), Sa)
    assert np.array_equal(np.concatenate([oa, ob], axis=1), o)
    assert np.array_equal(Sb, S)
    # and one decode step is one token of the recurrence
    od, Sd = decode_step(q[:, 0], k[:, 0], v[:, 0], ld[:, 0], e[:, 0], w[:, 0], S0)
    o1, S1 = recurrence(q[:, :1], k[:, :1], v[:, :1], ld[:, :1], e[:, :1], w[:, :1], S0)
    assert np.array_equal(od, o1[:, 0]) and np.array_equal(Sd, S1)


# P8 -- norm bound with a uniform erase (scalar beta in (0,1], ||k|| = 1): I - beta k k^T has
# spectral norm <= 1, so ||S_t||_F <= max_i a_{t,i} ||S_{t-1}||_F + beta_t ||v_t|| at every t
# (bounded memory norm, "KronLSTM ...", the mathematics section, as context).  For decoupled
# erase a single factor may expand, so there only a plateau over a long sequence is asserted.
def test_norm_bound_uniform_erase():
    q, k, v, ld, e, _, _ = _inputs(12, B=1, T=600, H=2, dk=16, dv=16, decay="channel", erase="head", write=None)
    _, _, states = recurrence(q, k, v, ld, e, None, None, return_states=True)
    nrm = np.linalg.norm(states, axis=(-2, -1))  # [B,H,T]
    prev = np.zeros(nrm.shape[:2])
    amax = np.exp(ld).max(axis=-1)  # [B,T,H]
    for t in range(q.shape[1]):
        bound = amax[:, t] * prev + e[:, t] * np.linalg.norm(v[:, t], axis=-1)
        assert np.all(nrm[:, :, t] <= bound * (1 + 1e-12) + 1e-12)
        prev = nrm[:, :, t]


def test_decoupled_factor_can_expand_and_state_plateaus():
    k = np.array([1.0, 1.0]) / np.sqrt(2.0)
    F = np.eye(2) - np.outer(np.array([1.0, 0.0]) * k, k)
    assert abs(np.linalg.norm(F, 2) - 1.1441228) < 1e-6
    q, k, v, ld, e, w, _ = _inputs(13, B=1, T=4000, H=1, dk=16, dv=16)
    _, _, states = recurrence(q, k, v, ld, e, w, None, return_states=True)
    nrm = np.linalg.norm(states[0, 0], axis=(-2, -1))
    T = nrm.shape[0]
    assert nrm[3 * T // 4:].max() <= 1.5 * nrm[T // 4: T // 2].max()


# P11 -- dk = dv = 1: s_t = a_t (1 - e_t k_t^2) s_{t-1} + k_t w_t v_t, o_t = q_t s_t.
def test_scalar_closed_form_d1():
    r = _rng(14)
    T = 40
    q, k, v = r.standard_normal(T), r.standard_normal(T), r.standard_normal(T)
    la, e, w = -np.log1p(np.exp(r.normal(-1, 1, T))), _sig(r.standard_normal(T)), _sig(r.standard_normal(T))
    s, ref = 0.7, []
    for t in range(T):
        s = np.exp(la[t]) * (1 - e[t] * k[t] ** 2) * s + k[t] * w[t] * v[t]
        ref.append(q[t] * s)
    W = lambda x: x[None, :, None, None]
    o, S = recurrence(W(q), W(k), W(v), W(la), W(e), W(w), np.full((1, 1, 1, 1), 0.7))
    assert np.allclose(o[0, :, 0, 0], ref, rtol=1e-13, atol=1e-14)
    assert abs(S[0, 0, 0, 0] - s) < 1e-13


# P10 -- an independently derived algorithm, the chunked WY/UT form (tests/chunk_model.py),
# equals the token loop for every chunk size and variant.
@pytest.mark.parametrize("chunk", [1, 7, 16, 64, 256])
@pytest.mark.parametrize("variant", ["scalar", "kda", "decoupled"])
def test_chunk_form_matches_token_loop(chunk, variant):
    args = {
        "scalar": dict(decay="head", erase="head", write=None),
        "kda": dict(decay="channel", erase="head", write=None),
        "decoupled": dict(decay="channel", erase="channel", write="channel"),
    }[variant]
    q, k, v, ld, e, w, S0 = _inputs(15, B=1, T=200, H=1, dk=16, dv=12, **args)
    o, S = recurrence(q, k, v, ld, e, w, S0)
    sel = lambda x: None if x is None else x[0, :, 0]
    oc, Sc = chunk_forward(sel(q), sel(k), sel(v), sel(ld), sel(e), sel(w), S0[0, 0], chunk=chunk)
    assert np.max(np.abs(oc - o[0, :, 0])) <= 1e-12 * np.max(np.abs(o))
    assert np.max(np.abs(Sc - S[0, 0])) <= 1e-12 * np.max(np.abs(S))
    if variant != "decoupled":  # the symmetric WY form must also agree with the general one
        oc2, Sc2 = chunk_forward(sel(q), sel(k), sel(v), sel(ld), sel(e), None, S0[0, 0], chunk=chunk, symmetric=False)
        assert np.max(np.abs(oc2 - oc)) <= 1e-12 * np.max(np.abs(o))


# A planted mistake must be caught: if the decay were applied after the erase (or the output
# read the state before the write) the explicit KDA form above would disagree.
def test_pins_catch_planted_mistakes():
    r = _rng(16)
    T, d = 9, 4
    q, v, k = r.standard_normal((T, d)), r.standard_normal((T, d)), _unit(r.standard_normal((T, d)))
    a = np.exp(-np.log1p(np.exp(r.normal(-1, 1, (T, d)))))
    beta = _sig(r.standard_normal(T))
    I = np.eye(d)
    S_true, S_wrong_order = np.zeros((d, d)), np.zeros((d, d))
    for t in range(T):
        S_true = (I - beta[t] * np.outer(k[t], k[t])) @ np.diag(a[t]) @ S_true + beta[t] * np.outer(k[t], v[t])
        S_wrong_order = np.diag(a[t]) @ (I - beta[t] * np.outer(k[t], k[t])) @ S_wrong_order + beta[t] * np.outer(k[t], v[t])
    wrap = lambda x: x[None, :, None]
    _, S = recurrence(wrap(q), wrap(k), wrap(v), wrap(np.log(a)), wrap(beta), None, None)
    assert np.allclose(S[0, 0], S_true, atol=1e-12)
    assert not np.allclose(S[0, 0], S_wrong_order, atol=1e-6)


# ---- packed sequences of different lengths -------------------------------------------------
# Each sequence is its own recurrence from its own initial state ("Gated DeltaNet-2 ...", the
# attention bottleneck: one fixed-size state per sequence, constant-memory decoding).


def _packed(seed, lens, H=2, dk=5, dv=4, decay="channel", erase="channel", write="channel", s0=True):
    q, k, v, ld, e, w, _ = _inputs(seed, B=1, T=int(sum(lens)), H=H, dk=dk, dv=dv, decay=decay,
                                   erase=erase, write=write, s0=False)
    S0 = _rng(seed + 1000).standard_normal((len(lens), H, dk, dv)) if s0 else None
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    return q, k, v, ld, e, w, S0, cu


# V1 -- equal lengths: the packed batch is the dense batch [N, L] reshaped.
@pytest.mark.parametrize("write", ["channel", None])
def test_varlen_equal_lengths_is_dense_batch(write):
    N, L = 3, 7
    q, k, v, ld, e, w, S0, cu = _packed(21, [L] * N, erase="channel" if write else "head", write=write)
    o, S = recurrence_varlen(q, k, v, ld, e, w, S0, cu)
    dense = lambda x: None if x is None else x.reshape((N, L) + x.shape[2:])
    od, Sd = recurrence(dense(q), dense(k), dense(v), dense(ld), dense(e), dense(w), S0)
    assert np.allclose(o.reshape(od.shape), od, rtol=0, atol=1e-13)
    assert np.allclose(S, Sd, rtol=0, atol=1e-13)


# V2 -- isolation: changing every input of one sequence leaves the others' outputs and states
# exactly as they were, and that sequence alone equals the single-sequence recurrence.
def test_varlen_sequences_are_isolated():
    lens = [4, 9, 1, 6]
    q, k, v, ld, e, w, S0, cu = _packed(22, lens)
    o, S = recurrence_varlen(q, k, v, ld, e, w, S0, cu)
    lo, hi = cu[1], cu[2]
    q2, v2 = q.copy(), v.copy()
    q2[:, lo:hi] += 1.0
    v2[:, lo:hi] *= -3.0
    S02 = S0.copy()
    S02[1] += 5.0
    o2, S2 = recurrence_varlen(q2, k, v2, ld, e, w, S02, cu)
    keep = np.ones(q.shape[1], bool)
    keep[lo:hi] = False
    assert np.array_equal(o2[:, keep], o[:, keep])
    assert np.array_equal(S2[[0, 2, 3]], S[[0, 2, 3]])
    assert not np.allclose(o2[:, lo:hi], o[:, lo:hi])
    cut = lambda x: x[:, lo:hi]
    o1, S1 = recurrence(cut(q2), cut(k), cut(v2), cut(ld), cut(e), cut(w), S02[1:2])
    assert np.array_equal(o2[:, lo:hi], o1) and np.array_equal(S2[1], S1[0])


# V3 -- empty sequences (at the start, in the middle, at the end) pass their initial state
# through unchanged (zeros without one) and do not shift their neighbours' tokens.
@pytest.mark.parametrize("s0", [True, False])
def test_varlen_empty_sequences(s0):
    lens = [0, 5, 0, 0, 3, 0]
    q, k, v, ld, e, w, S0, cu = _packed(23, lens, s0=s0)
    o, S = recurrence_varlen(q, k, v, ld, e, w, S0, cu)
    for n in (0, 2, 3, 5):
        assert np.array_equal(S[n], S0[n] if s0 else np.zeros_like(S[n]))
    nz = [1, 4]
    o_ref, S_ref = recurrence_varlen(q, k, v, ld, e, w, None if S0 is None else S0[nz],
                                     np.array([0, 5, 8], np.int32))
    assert np.array_equal(o, o_ref) and np.array_equal(S[nz], S_ref)


# V4 -- split invariance, the prefill-to-decode handoff: one sequence cut into two packed
# sequences, the second started from the first one's final state, gives the uncut outputs;
# decode steps continued from a packed prefill's states equal the longer prefill.
def test_varlen_split_and_decode_handoff():
    q, k, v, ld, e, w, S0, _ = _packed(24, [10], H=2)
    o, S = recurrence_varlen(q, k, v, ld, e, w, S0, np.array([0, 10], np.int32))
    oa, Sa = recurrence_varlen(q[:, :6], k[:, :6], v[:, :6], ld[:, :6], e[:, :6], w[:, :6], S0,
                               np.array([0, 6], np.int32))
    ob, Sb = recurrence_varlen(q[:, 6:], k[:, 6:], v[:, 6:], ld[:, 6:], e[:, 6:], w[:, 6:], Sa,
                               np.array([0, 4], np.int32))
    assert np.array_equal(np.concatenate([oa, ob], axis=1), o) and np.array_equal(Sb, S)
    # two sequences: prefill 4 and 7 tokens, then decode 3 more of each
    lens, extra = [4, 7], 3
    qs, ks, vs, lds, es, ws, S0s, _ = _packed(25, [sum(lens) + 2 * extra], H=2)
    S0s = _rng(26).standard_normal((2, 2, 5, 4))
    seqs = [(0, 4 + extra), (4 + extra, 4 + extra + 7 + extra)]
    take = lambda x, lo, hi: x[:, lo:hi]
    pre = np.concatenate([np.arange(lo, lo + L) for (lo, _), L in zip(seqs, lens)])
    cu = np.array([0, lens[0], sum(lens)], np.int32)
    _, Sp = recurrence_varlen(*(x[:, pre] for x in (qs, ks, vs, lds, es, ws)), S0s, cu)
    for j in range(extra):
        idx = [lo + L + j for (lo, _), L in zip(seqs, lens)]
        od, Sp = decode_step(*(x[0, idx] for x in (qs, ks, vs, lds, es, ws)), Sp)
        for n, (lo, hi) in enumerate(seqs):
            o_full, _ = recurrence(*(take(x, lo, lo + lens[n] + j + 1) for x in (qs, ks, vs, lds, es, ws)),
                                   S0s[n:n + 1])
            assert np.allclose(od[n], o_full[0, -1], rtol=0, atol=1e-12)


# V5 -- one-token sequences from a zero state, closed form: S = k (w * v)^T and
# o = (q . k) (w * v), each from its own token only.
def test_varlen_one_token_closed_form():
    lens = [1, 1, 1]
    q, k, v, ld, e, w, _, cu = _packed(27, lens, s0=False)
    o, S = recurrence_varlen(q, k, v, ld, e, w, None, cu)
    for n in range(3):
        kn, qn, vw = k[0, n], q[0, n], w[0, n] * v[0, n]  # [H, d]
        assert np.allclose(S[n], kn[:, :, None] * vw[:, None, :], rtol=0, atol=1e-14)
        assert np.allclose(o[0, n], np.sum(qn * kn, -1)[:, None] * vw, rtol=0, atol=1e-14)


def test_varlen_rejects_bad_offsets():
    q, k, v, ld, e, w, S0, cu = _packed(28, [3, 2])
    for bad in ([0, 3], [1, 3, 5], [0, 4, 3]):
        with pytest.raises(ValueError):
            recurrence_varlen(q, k, v, ld, e, w, None, np.array(bad, np.int32))


# ---- FG2-GDN's per-channel rate, absorbed as sqrt(beta) into key and value -------------------
# ("FG2-GDN ...", section 2, FG2-GDN update rule)


# F1 -- the explicit form (I - k~ k~^T) Diag(a) S + k~ v~^T as dense matrix products, channel and
# scalar decay.
@pytest.mark.parametrize("decay", ["channel", "head"])
def test_fg2_explicit_matrix_form(decay):
    r = _rng(41)
    T, d = 17, 6
    q, k, v = r.standard_normal((T, d)), _unit(r.standard_normal((T, d))), r.standard_normal((T, d))
    la = -np.log1p(np.exp(r.normal(-2, 1, (T, d) if decay == "channel" else (T,))))
    beta = _sig(r.standard_normal((T, d)))
    S0 = r.standard_normal((d, d))
    I = np.eye(d)
    S = S0.copy()
    o_ref = np.empty((T, d))
    for t in range(T):
        kt, vt = np.sqrt(beta[t]) * k[t], np.sqrt(beta[t]) * v[t]
        A = np.diag(np.exp(la[t]) * np.ones(d))
        S = (I - np.outer(kt, kt)) @ A @ S + np.outer(kt, vt)
        o_ref[t] = S.T @ q[t]
    wrap = lambda x: x[None, :, None]
    o, S_out = recurrence_fg2(wrap(q), wrap(k), wrap(v), wrap(la), wrap(beta), S0[None, None])
    assert np.allclose(o[0, :, 0], o_ref, rtol=0, atol=1e-12 * np.abs(o_ref).max())
    assert np.allclose(S_out[0, 0], S, rtol=0, atol=1e-12 * np.abs(S).max())


# F2 -- a rate that is the same on every channel is KDA's scalar beta: sqrt(b) k sqrt(b) k^T =
# b k k^T and sqrt(b) k sqrt(b) v^T = b k v^T.
def test_fg2_constant_rate_is_kda():
    q, k, v, ld, e, _, S0 = _inputs(42, B=2, T=15, H=2, dk=5, dv=5, decay="channel", erase="head", write=None)
    beta = np.repeat(e[..., None], 5, axis=-1)
    o1, S1 = recurrence_fg2(q, k, v, ld, beta, S0)
    o2, S2 = recurrence(q, k, v, ld, e, None, S0)
    assert np.allclose(o1, o2, rtol=0, atol=1e-12) and np.allclose(S1, S2, rtol=0, atol=1e-12)
    # and a rate that differs between channels does not reduce to any scalar one
    beta2 = beta.copy()
    beta2[..., 0] *= 0.5
    o3, _ = recurrence_fg2(q, k, v, ld, beta2, S0)
    assert not np.allclose(o3, o2, atol=1e-6)


# F3 -- the online-learning reading: with no decay, one step is the gradient step
# S <- S - k~ (k~^T S - v~^T) on 1/2 ||S^T k~ - v~||^2 (a diagonal learning-rate matrix on the
# original pair), so the new state reads back k~^T S_new = (1 - ||k~||^2) k~^T S + ||k~||^2 v~^T.
def test_fg2_readback_identity():
    r = _rng(43)
    d = 7
    q, k, v = r.standard_normal(d), _unit(r.standard_normal(d)), r.standard_normal(d)
    beta = _sig(r.standard_normal(d))
    S0 = r.standard_normal((d, d))
    wrap = lambda x: x[None, None, None]
    _, S = recurrence_fg2(wrap(q), wrap(k), wrap(v), wrap(np.zeros(d)), wrap(beta), S0[None, None])
    kt, vt = np.sqrt(beta) * k, np.sqrt(beta) * v
    n2 = kt @ kt
    assert np.allclose(kt @ S[0, 0], (1 - n2) * (kt @ S0) + n2 * vt, rtol=0, atol=1e-12)


# ---- gradients (recurrence_bwd) -------------------------------------------------------------


def _bwd_case(seed, decay, erase, write, B=2, T=9, H=2, dk=4, dv=3):
    q, k, v, ld, e, w, S0 = _inputs(seed, B=B, T=T, H=H, dk=dk, dv=dv, decay=decay, erase=erase, write=write)
    r = _rng(seed + 500)
    dO = r.standard_normal(q.shape[:3] + (dv,))
    dST = r.standard_normal(S0.shape)
    return dict(q=q, k=k, v=v, log_decay=ld, erase=e, write=w, S0=S0), dO, dST


def _loss(x, dO, dST):
    o, S = recurrence(x["q"], x["k"], x["v"], x["log_decay"], x["erase"], x["write"], x["S0"])
    return float(np.sum(o * dO) + np.sum(S * dST))


GRAD_KEY = dict(q="dq", k="dk", v="dv", log_decay="dlog_decay", erase="derase", write="dwrite", S0="dS0")
BWD_VARIANTS = [("head", "head", None), ("channel", "head", None), ("channel", "channel", "channel"),
                ("head", "channel", "head"), ("channel", "channel", None)]


# G1 -- central finite differences of the forward along a random direction of every input
# agree with the adjoint's directional derivative <grad, d>.
@pytest.mark.parametrize("decay,erase,write", BWD_VARIANTS)
def test_bwd_matches_finite_differences(decay, erase, write):
    dv = 4 if (erase == "channel" and write is None) else 3
    x, dO, dST = _bwd_case(51, decay, erase, write, dv=dv)
    g = recurrence_bwd(**x, dO=dO, dS_T=dST)
    r = _rng(52)
    h = 1e-6
    for name, val in x.items():
        if val is None:
            continue
        d = r.standard_normal(val.shape)
        xp, xm = dict(x), dict(x)
        xp[name], xm[name] = val + h * d, val - h * d
        fd = (_loss(xp, dO, dST) - _loss(xm, dO, dST)) / (2 * h)
        an = float(np.sum(g[GRAD_KEY[name]] * d))
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (name, fd, an)


# G2 -- torch autograd through a torch forward written here with plain tensor ops (float64)
# gives the same gradients to rounding.
@pytest.mark.parametrize("decay,erase,write", BWD_VARIANTS)
def test_bwd_matches_autograd(decay, erase, write):
    import torch

    dv = 4 if (erase == "channel" and write is None) else 3
    x, dO, dST = _bwd_case(53, decay, erase, write, dv=dv)
    g = recurrence_bwd(**x, dO=dO, dS_T=dST)
    tx = {n: (None if val is None else torch.tensor(val, dtype=torch.float64, requires_grad=True)) for n, val in x.items()}
    q, k, v, S = tx["q"], tx["k"], tx["v"], tx["S0"]
    a = torch.exp(tx["log_decay"])
    e = tx["erase"]
    w = tx["write"] if tx["write"] is not None else tx["erase"]
    outs = []
    for t in range(q.shape[1]):
        at = a[:, t] if a.dim() == 4 else a[:, t, :, None]
        et = e[:, t] if e.dim() == 4 else e[:, t, :, None]
        wt = w[:, t] if w.dim() == 4 else w[:, t, :, None]
        kt, vt, qt = k[:, t], v[:, t], q[:, t]
        Sp = at[..., :, None] * S
        m = torch.einsum("bhi,bhij->bhj", kt, Sp)
        S = Sp - torch.einsum("bhi,bhj->bhij", et * kt, m) + torch.einsum("bhi,bhj->bhij", kt, wt * vt)
        outs.append(torch.einsum("bhij,bhi->bhj", S, qt))
    o = torch.stack(outs, 1)
    L = (o * torch.tensor(dO)).sum() + (S * torch.tensor(dST)).sum()
    names = [n for n in tx if tx[n] is not None]
    grads = torch.autograd.grad(L, [tx[n] for n in names])
    for n, gr in zip(names, grads):
        ref = gr.numpy()
        got = g[GRAD_KEY[n]]  # a shared erase/write gate: autograd sums both uses, as the adjoint does
        assert np.allclose(got, ref, rtol=0, atol=1e-12 * max(1.0, np.abs(ref).max())), n


# G3 -- with no erase and no decay the recurrence is causal linear attention, whose gradient in
# q is closed-form: dq_t = S0 dO_t + sum_{s <= t} k_s (w_s v_s . dO_t).
def test_bwd_linear_attention_closed_form():
    x, dO, dST = _bwd_case(54, "head", "head", "head")
    x["erase"] = np.zeros_like(x["erase"])
    x["log_decay"] = np.zeros_like(x["log_decay"])
    g = recurrence_bwd(**x, dO=dO, dS_T=dST)
    q, k, v, w, S0 = x["q"], x["k"], x["v"], x["write"], x["S0"]
    B, T, H, _ = q.shape
    ref = np.empty_like(q)
    for b in range(B):
        for h in range(H):
            for t in range(T):
                acc = S0[b, h] @ dO[b, t, h]
                for s in range(t + 1):
                    acc = acc + k[b, s, h] * (w[b, s, h] * v[b, s, h] @ dO[b, t, h])
                ref[b, t, h] = acc
    assert np.allclose(g["dq"], ref, rtol=0, atol=1e-12)


# G4 -- FG2's rate form: central finite differences of recurrence_fg2 along random directions
# of q, k, v, the decay, the rate and S0 agree with recurrence_fg2_bwd.
@pytest.mark.parametrize("decay", ["channel", "head"])
def test_fg2_bwd_matches_finite_differences(decay):
    r = _rng(61)
    B, T, H, d = 2, 8, 2, 4
    x = dict(q=r.standard_normal((B, T, H, d)), k=_unit(r.standard_normal((B, T, H, d))),
             v=r.standard_normal((B, T, H, d)),
             log_decay=-np.log1p(np.exp(r.normal(-2, 1, (B, T, H, d) if decay == "channel" else (B, T, H)))),
             beta=_sig(r.standard_normal((B, T, H, d))), S0=r.standard_normal((B, H, d, d)))
    dO, dST = r.standard_normal((B, T, H, d)), r.standard_normal((B, H, d, d))
    g = recurrence_fg2_bwd(**x, dO=dO, dS_T=dST)
    key = dict(q="dq", k="dk", v="dv", log_decay="dlog_decay", beta="dbeta", S0="dS0")

    def loss(y):
        o, S = recurrence_fg2(**y)
        return float(np.sum(o * dO) + np.sum(S * dST))

    h = 1e-6
    for name, val in x.items():
        dirn = r.standard_normal(val.shape)
        yp, ym = dict(x), dict(x)
        yp[name], ym[name] = val + h * dirn, val - h * dirn
        fd = (loss(yp) - loss(ym)) / (2 * h)
        an = float(np.sum(g[key[name]] * dirn))
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (name, fd, an)
