"""fp64 chunk-form model of the recurrence (test-side design model, not the oracle).

The chunked forward that the pages describe keeps the rank-1 Householder structure of each
token step so that a chunk of steps folds into dense matrix products (WY/UT representation,
"FG2-GDN ...", section 2, "preserving symmetry"; diagonal-plus-low-rank compatibility with
chunked parallel training, section 3), and rebuilds the in-chunk states from the chunk's
boundary state ("Linearized 2-Simplicial Attention", Method, architecture and implementation).

For one chunk with local tokens t = 1..C, incoming state S0 and chunk-local cumulative
log-decay g_t = sum_{i<=t} log a_i:
  K+ rows k_t e^{g_t}, Q+ rows q_t e^{g_t}, K- rows k_i e^{-g_i}, U- rows u_i e^{-g_i},
  Kend rows k_i e^{g_C - g_i}, Uend rows u_i e^{g_C - g_i},  u = e * k, vt = w * v
  A_kk = strict_lower(K+ K-^T), A_ku = strict_lower(K+ U-^T),
  A_qk = lower(Q+ K-^T),        A_qu = lower(Q+ U-^T)
  M    = (I + A_ku)^{-1} (K+ S0 + A_kk Vt)         (rows m_t = (Diag(a_t) S_{t-1})^T k_t)
  O    = Q+ S0 + A_qk Vt - A_qu M
  S_C  = Diag(e^{g_C}) S0 + Kend^T Vt - Uend^T M
With one scalar beta for erase and write (u = beta k, vt = beta v) this becomes the
symmetric WY form:  T = (I + Diag(beta) A_kk)^{-1},  delta = T Diag(beta) (V - K+ S0),
O = Q+ S0 + A_qk delta,  S_C = Diag(e^{g_C}) S0 + Kend^T delta.

This module is used only by the tests: it checks the oracle against an independently derived
algorithm (chunk size 1 ... 256 must all agree with the token loop) and it fixes the exact
signs, masks and exponent references the HIP chunk kernel implements.
"""
from __future__ import annotations

import numpy as np


def _lower(x, strict):
    C = x.shape[-1]
    mask = np.tril(np.ones((C, C)), -1 if strict else 0)
    return x * mask


def chunk_forward(q, k, v, log_decay, erase, write=None, S0=None, chunk=64, symmetric=None):
    """Chunked evaluation of the recurrence for a single (b, h): q, k [T, dk], v [T, dv],
    gates [T] or [T, d].  Returns (o [T, dv], S_T)."""
    q, k, v = (np.asarray(x, np.float64) for x in (q, k, v))
    T, dk = k.shape
    dv = v.shape[1]
    la = np.asarray(log_decay, np.float64)
    la = np.broadcast_to(la[:, None] if la.ndim == 1 else la, (T, dk))
    e = np.asarray(erase, np.float64)
    scalar_beta = e.ndim == 1 and write is None
    e = np.broadcast_to(e[:, None] if e.ndim == 1 else e, (T, dk))
    if write is None:
        w = np.asarray(erase, np.float64)
    else:
        w = np.asarray(write, np.float64)
    w = np.broadcast_to(w[:, None] if w.ndim == 1 else w, (T, dv))
    if symmetric is None:
        symmetric = scalar_beta
    S = np.zeros((dk, dv)) if S0 is None else np.array(S0, np.float64)
    o = np.zeros((T, dv))
    for c0 in range(0, T, chunk):
        sl = slice(c0, min(c0 + chunk, T))
        C = sl.stop - sl.start
        g = np.cumsum(la[sl], axis=0)  # chunk-local, [C, dk]
        gC = g[-1]
        kc, qc, vc = k[sl], q[sl], v[sl]
        Kp, Qp = kc * np.exp(g), qc * np.exp(g)
        Km = kc * np.exp(-g)
        Kend = kc * np.exp(gC - g)
        A_kk = _lower(Kp @ Km.T, True)
        A_qk = _lower(Qp @ Km.T, False)
        if symmetric:
            beta = np.asarray(erase, np.float64)[sl]
            Tm = np.linalg.inv(np.eye(C) + beta[:, None] * A_kk)
            delta = Tm @ (beta[:, None] * (vc - Kp @ S))
            o[sl] = Qp @ S + A_qk @ delta
            S = np.exp(gC)[:, None] * S + Kend.T @ delta
        else:
            u = e[sl] * kc
            Vt = w[sl] * vc
            Um = u * np.exp(-g)
            Uend = u * np.exp(gC - g)
            A_ku = _lower(Kp @ Um.T, True)
            A_qu = _lower(Qp @ Um.T, False)
            M = np.linalg.solve(np.eye(C) + A_ku, Kp @ S + A_kk @ Vt)
            o[sl] = Qp @ S + A_qk @ Vt - A_qu @ M
            S = np.exp(gC)[:, None] * S + Kend.T @ Vt - Uend.T @ M
    return o, S
