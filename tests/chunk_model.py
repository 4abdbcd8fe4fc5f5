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


# ------------------------------------------------------------------------------------------
# Kernel-faithful emulation of the matrix-core chunk path.
#
# The chunk form above is exact in any arithmetic with unbounded range; the HIP kernels run its
# products on fp16 matrix operands (fp32 accumulation, fp32 state), so every decay factor that
# multiplies an operand must stay inside fp16's range, and the way each factor e^{g_t - g_i} is
# split between the two operands of a product (its reference point) decides whether the
# method stays exact for every valid decay a in (0, 1).  `kernel_emulation` reproduces the
# roundings and the referencing of one scheme in fp64:
#
#   scheme="safe"      every factor that is not immediately followed by its exact inverse is
#                      e^{x} with x <= 0: the state is referenced at the chunk start (rows
#                      q_t e^{g_t}, k_t e^{g_t}; state update k_i e^{g_C - g_i}), the
#                      off-diagonal 16 x 16 blocks of the Gram matrices at their block
#                      boundary, and the diagonal blocks either at the block's log-midpoint
#                      (when its decay is at most 12 nats on every channel, so both factors lie
#                      within e^{+-6}) or, beyond that, by levels: pairs split at the boundary of
#                      the halves of 16-, 8-, 4- and 2-token segments, plus the diagonal.
#   scheme="midpoint"  the referencing of the first kernel version: every operand taken
#                      relative to the chunk's midpoint, with exponents clamped at 11 and the
#                      state scaled by e^{g_mid} into fp16 -- exact only while half a chunk's
#                      log-decay stays above -11.
#
# fp16 rounding is applied wherever the kernel stores or feeds an fp16 matrix operand; sums
# are kept in fp64 (the kernel accumulates in fp32, which is far finer than fp16 operands).
# ------------------------------------------------------------------------------------------
_BLK = 16
_FAST_SPAN = 12.0  # largest per-channel log-decay over a 16-token block for the midpoint split
_FP16_SAFE = 32768.0


def _h(x):
    """Round to fp16 (round to nearest even; overflow gives inf, as the conversion does)."""
    with np.errstate(over="ignore"):
        return np.asarray(x, np.float64).astype(np.float16).astype(np.float64)


def _diag_block(rows, cols, gl, D):
    """Diagonal 16 x 16 block of the Gram matrices, A[x][y][t, i] = sum_d rows[x][t, d] cols[y][i, d]
    e^{gl[t, d] - gl[i, d]} for i <= t (lower triangle, diagonal included; the caller masks).

    rows: dict name -> [16, d] row operands (k, q); cols: dict name -> [16, d] column operands
    (k, u); gl: [16, d] in-block inclusive prefix of the log-decay; D: [d] block total."""
    n = gl.shape[0]
    lower = np.tril(np.ones((n, n)))
    out = {}
    half = D / 2
    ops_r = {x: _h(r * np.exp(gl - half)) for x, r in rows.items()}
    ops_c = {y: _h(c * np.exp(half - gl)) for y, c in cols.items()}
    fast = bool(np.all(D >= -_FAST_SPAN))
    for dct in (ops_r, ops_c):
        for a in dct.values():
            fast = fast and bool(np.all(np.isfinite(a)) and np.all(np.abs(a) <= _FP16_SAFE))
    if fast:
        for x in rows:
            for y in cols:
                out[x, y] = (ops_r[x] @ ops_c[y].T) * lower
        return out, True
    # levels: segments of s tokens, rows in the second half, columns in the first, both
    # referenced at the last token of the first half (every factor e^{x}, x <= 0)
    p = np.arange(n)
    for x in rows:
        for y in cols:
            out[x, y] = np.zeros((n, n))
    s = n
    while s >= 2:
        hs = s // 2
        seg, pos = p // s, p % s
        ref = seg * s + hs - 1
        is_row = pos >= hs
        f = np.where(is_row[:, None], np.exp(gl - gl[ref]), np.exp(gl[ref] - gl))
        same = (seg[:, None] == seg[None, :]) & is_row[:, None] & ~is_row[None, :]
        for x, r in rows.items():
            ro = _h(np.where(is_row[:, None], r * f, 0.0))
            for y, c in cols.items():
                co = _h(np.where(is_row[:, None], 0.0, c * f))
                out[x, y] += np.where(same, ro @ co.T, 0.0)
        s = hs
    eye = np.eye(n, dtype=bool)
    for x, r in rows.items():
        for y, c in cols.items():
            out[x, y] += np.where(eye, _h(r) @ _h(c).T, 0.0)
    return out, False


def _gram_safe(rows, cols, gl, D):
    """Lower-triangular C x C Gram matrices with block-boundary referencing (see above).
    rows/cols: dict name -> [C, d]; gl: [C, d] in-block prefixes; D: [nblk, d] block totals.
    Returns (dict (x, y) -> [C, C] with the diagonal included, list of fast flags per block)."""
    C = gl.shape[0]
    nb = (C + _BLK - 1) // _BLK
    A = {(x, y): np.zeros((C, C)) for x in rows for y in cols}
    fast = []
    # column operands referenced at the end of their own block: k_i e^{D_J - gl_i} <= 1
    cend = {y: _h(c * np.exp(D[np.arange(C) // _BLK] - gl)) for y, c in cols.items()}
    for I in range(nb):
        ti = slice(_BLK * I, min(_BLK * (I + 1), C))
        rop = {x: _h(r[ti] * np.exp(gl[ti])) for x, r in rows.items()}  # e^{g_t - g_{b_I}}
        for J in range(I):
            tj = slice(_BLK * J, _BLK * (J + 1))
            # the decay of the blocks strictly between J and I, applied in fp16 to the
            # stored column fragment
            F = _h(np.exp(D[J + 1:I].sum(axis=0))) if I > J + 1 else None
            for y in cols:
                co = cend[y][tj] if F is None else _h(cend[y][tj] * F)
                for x in rows:
                    A[x, y][ti, tj] = rop[x] @ co.T
        blk, ok = _diag_block({x: r[ti] for x, r in rows.items()}, {y: c[ti] for y, c in cols.items()},
                              gl[ti], D[I])
        fast.append(ok)
        for key, val in blk.items():
            A[key][ti, ti] = val
    return A, fast


def _tri(x, strict):
    return np.tril(x, -1 if strict else 0)


def kernel_emulation(q, k, v, log_decay, erase, write=None, S0=None, scheme="safe", fg2=False,
                     return_flags=False):
    """Emulate the matrix-core chunk path for one (b, h); arguments as ``chunk_forward`` plus
    ``fg2`` (erase is then FG2-GDN's per-channel rate beta, taken as sqrt(beta) into k and v with
    unit gates).  Returns (o [T, dv], S_T) in fp64, or with ``return_flags`` also the list of
    per-block fast-path flags of the safe scheme."""
    C = 64
    q, k, v = (np.asarray(x, np.float64) for x in (q, k, v))
    T, dk = k.shape
    dv = v.shape[1]
    la = np.asarray(log_decay, np.float64)
    dch = la.ndim == 2
    la = np.broadcast_to(la[:, None] if la.ndim == 1 else la, (T, dk))
    e_in = np.asarray(erase, np.float64)
    if fg2:
        sq = np.sqrt(e_in)
        k = k * sq
        v = _h(v * sq)  # the prep writes v~ into the packet in fp16
        e = np.ones((T, dk))
        w = np.ones((T, dv))
        symmetric, beta = True, np.ones(T)
    else:
        symmetric = e_in.ndim == 1 and write is None
        e = np.broadcast_to(e_in[:, None] if e_in.ndim == 1 else e_in, (T, dk))
        w_in = e_in if write is None else np.asarray(write, np.float64)
        w = np.broadcast_to(w_in[:, None] if w_in.ndim == 1 else w_in, (T, dv))
        beta = e_in if symmetric else None
    S = np.zeros((dk, dv)) if S0 is None else np.array(S0, np.float64)
    o = np.zeros((T, dv))
    flags = []
    scalar_path = symmetric and not dch  # plain k, q tiles with per-row / per-element factors
    for c0 in range(0, T, C):
        n = min(C, T - c0)
        sl = slice(c0, c0 + n)
        pad = lambda x: np.concatenate([x, np.zeros((C - n,) + x.shape[1:])]) if n < C else x
        kc, qc, vc = pad(k[sl]), pad(q[sl]), pad(v[sl])
        lac, ec, wc = pad(la[sl]), pad(e[sl]), pad(w[sl])
        g = np.cumsum(lac, axis=0)
        gC = g[-1]
        gm = g[31]
        if symmetric:
            bc = pad(np.asarray(beta, np.float64)[sl])
        if scheme == "safe":
            blocks = np.arange(C) // _BLK
            D = np.stack([lac[_BLK * b:_BLK * (b + 1)].sum(axis=0) for b in range(C // _BLK)])
            gb = np.concatenate([np.zeros((1, dk)), np.cumsum(D, axis=0)[:-1]])
            gl = g - gb[blocks]
        if scalar_path:
            # plain fp16 k, q; Gram products take e^{g_t - g_i} <= 1 per element in fp32
            kh, qh = _h(kc), _h(qc)
            gs = g[:, 0]
            dec = np.exp(np.minimum(gs[:, None] - gs[None, :], 0.0))
            A_kk = _tri((kh @ kh.T) * dec, True)
            A_qk = _tri((qh @ kh.T) * dec, False)
            if scheme == "safe":
                St, fp, fm, fcm = _h(S), np.exp(gs), np.exp(gC[0] - gs), 1.0
            else:
                St = _h(np.exp(gm[0]) * S)
                fp = np.exp(np.minimum(gs - gm[0], 11.0))
                fm = np.exp(np.minimum(gm[0] - gs, 11.0))
                fcm = np.exp(min(gC[0] - gm[0], 11.0))
            Tm = _h(np.linalg.inv(np.eye(C) + bc[:, None] * A_kk))
            Aq = _h(A_qk)
            XK = (kh @ St) * fp[:, None]
            XQ = (qh @ St) * fp[:, None]
            R = _h(bc[:, None] * (vc - XK))
            delta = Tm @ R
            dh = _h(delta)
            O = XQ + Aq @ dh
            S = np.exp(gC[0]) * S + fcm * (kh.T @ _h(delta * fm[:, None]))
            o[sl] = O[:n]
            continue
        u = ec * kc
        rows = {"k": kc, "q": qc}
        cols = {"k": kc} if symmetric else {"k": kc, "u": u}
        if scheme == "safe":
            A, fl = _gram_safe(rows, cols, gl, D)
            flags.extend(fl)
            Kp, Qp = _h(kc * np.exp(g)), _h(qc * np.exp(g))
            Kend = _h(kc * np.exp(gC - g))
            Uend = _h(u * np.exp(gC - g))
            St = _h(S)
            fcm = 1.0
        else:
            fpm = np.exp(np.minimum(g - gm, 11.0))
            fmm = np.exp(np.minimum(gm - g, 11.0))
            Kp, Qp = _h(kc * fpm), _h(qc * fpm)
            Km, Um = _h(kc * fmm), _h(u * fmm)
            A = {("k", "k"): Kp @ Km.T, ("q", "k"): Qp @ Km.T, ("k", "u"): Kp @ Um.T, ("q", "u"): Qp @ Um.T}
            St = _h(np.exp(gm)[:, None] * S)
            Kend, Uend = Km, Um
            fcm = np.exp(np.minimum(gC - gm, 11.0))[:, None]
        XK = Kp @ St
        XQ = Qp @ St
        if symmetric:
            Tm = _h(np.linalg.inv(np.eye(C) + bc[:, None] * _tri(A["k", "k"], True)))
            Aq = _h(_tri(A["q", "k"], False))
            R = _h(bc[:, None] * (vc - XK))
            dh = _h(Tm @ R)
            O = XQ + Aq @ dh
            S = np.exp(gC)[:, None] * S + fcm * (Kend.T @ dh)
        else:
            Tm = _h(np.linalg.inv(np.eye(C) + _tri(A["k", "u"], True)))
            Akk = _h(_tri(A["k", "k"], True))
            Aqk = _h(_tri(A["q", "k"], False))
            Aqu = _h(_tri(A["q", "u"], False))
            Vt = _h(wc * vc)
            Y = _h(XK + Akk @ Vt)
            Mh = _h(Tm @ Y)
            O = XQ + Aqk @ Vt - Aqu @ Mh
            S = np.exp(gC)[:, None] * S + fcm * (Kend.T @ Vt - Uend.T @ Mh)
        o[sl] = O[:n]
    if return_flags:
        return o, S, flags
    return o, S


# ------------------------------------------------------------------------------------------
# Chunk form of the gradients (the matrix-core backward's algebra), fp64.
#
# For one chunk, with S its incoming state, G the state's adjoint at its end and dO its output
# adjoint, the general (non-symmetric) chunk form above gives, by reverse mode through
#   M = (I + A_ku)^{-1} (K+ S + A_kk Vt),  O = Q+ S + A_qk Vt - A_qu M,
#   S_C = Diag(e^{g_C}) S + Kend^T Vt - Uend^T M:
#   Z     = -(I + A_ku)^{-T} (A_qu^T dO + Uend G)       (the adjoint of K+ S + A_kk Vt)
#   dK+   = Z S^T,  dQ+ = dO S^T,  dKend = Vt G^T,  dUend = -M G^T
#   dA_kk = strict(Z Vt^T), dA_ku = -strict(Z M^T), dA_qk = lower(dO Vt^T), dA_qu = -lower(dO M^T)
#   dVt   = A_kk^T Z + A_qk^T dO + Kend G,  dGamma = rowsum(S * G)
#   S's adjoint at the chunk start: Diag(e^{g_C}) G + Q+^T dO + K+^T Z   (the adjoint scan)
# and, through the Gram matrices A_xy[t, i] = sum_d x_t,d y_i,d e^{g_t,d - g_i,d}:
#   dx_t = sum_i dA[t, i] y_i e^{g_t - g_i},  dy_i = sum_t dA[t, i] x_t e^{g_t - g_i},
#   and the cumulative log-decay g takes x * dx on the row side and -y * dy on the column side.
# Every decayed operand adds its own share to g's adjoint (K+ = k e^{g}: + K+ * dK+; Kend =
# k e^{g_C - g}: - Kend * dKend at t and + at C), e^{g_C} adds e^{g_C} dGamma at C, and the
# log-decay's adjoint is the reverse prefix sum of g's over the chunk.
# With FG2's rate (u = k~, unit gates, T symmetric) A_ku = A_kk, A_qu = A_qk and Uend = Kend, so
# their adjoints merge: dA_kk = strict(Z Delta^T), dA_qk = lower(dO Delta^T), dKend = Delta G^T
# with Delta = Vt - M, and dVt = -Z.
# ------------------------------------------------------------------------------------------
def _masked_exp_diff(g, strict):
    """E[t, i, d] = e^{g_t,d - g_i,d} on the (strict) lower triangle, 0 elsewhere."""
    C = g.shape[0]
    mask = np.tril(np.ones((C, C), dtype=bool), -1 if strict else 0)
    diff = np.where(mask[:, :, None], g[:, None, :] - g[None, :, :], -np.inf)
    return np.exp(diff)


def gram_bwd_exact(dA, x, y, g, strict):
    """(dx, dy) of A = mask(x_t . y_i e^{g_t - g_i}) for the adjoint dA, element by element."""
    W = dA[:, :, None] * _masked_exp_diff(g, strict)
    return np.einsum("tid,id->td", W, y), np.einsum("tid,td->id", W, x)


def gram_bwd_blocked(dA, x, y, g, strict, blk=16, rnd=lambda a: a):
    """The same in the kernel's arrangement: diagonal blk x blk blocks element by element; an
    off-diagonal block (I, J), J < I, as one product dA_IJ Y~_J (and dA_IJ^T X~_I) of operands
    referenced inside their own block -- Y~ = y e^{g_r - g} with r the last token of J, X~ =
    x e^{g - g_s} with s the last token before I -- scaled by e^{g_s - g_r} per channel and by the
    row factor (e^{g_t - g_s} or e^{g_r - g_i}).  Every factor is e^{x} with x <= 0.  ``rnd``
    rounds the product operands (fp16 in the kernel)."""
    C = g.shape[0]
    nb = C // blk
    dx, dy = np.zeros_like(x), np.zeros_like(y)
    for b in range(nb):
        sl = slice(blk * b, blk * (b + 1))
        a, c = gram_bwd_exact(dA[sl, sl], x[sl], y[sl], g[sl], strict)
        dx[sl] += a
        dy[sl] += c
    dAr = rnd(dA)
    for I in range(1, nb):
        si = slice(blk * I, blk * (I + 1))
        s = blk * I - 1
        Xt = rnd(x[si] * np.exp(g[si] - g[s]))
        for J in range(I):
            sj = slice(blk * J, blk * (J + 1))
            r = blk * J + blk - 1
            F = np.exp(g[s] - g[r])
            Yt = rnd(y[sj] * np.exp(g[r] - g[sj]))
            dx[si] += np.exp(g[si] - g[s]) * F * (dAr[si, sj] @ Yt)
            dy[sj] += np.exp(g[r] - g[sj]) * F * (dAr[si, sj].T @ Xt)
    return dx, dy


def chunk_backward(q, k, v, log_decay, erase, write=None, S0=None, dO=None, dS_T=None, fg2=False,
                   blocked=False, fp16=False):
    """Gradients of one (b, h) through the chunk form (chunks of 64, the last one padded with
    zero inputs and unit decay, as the kernels do), in fp64: the forward stores every chunk's
    incoming state S and reads M (FG2: Delta = T (Vt - K+ S)), the adjoint scan every chunk's
    end adjoint G and Z, and each chunk's gradients follow from those alone.  Arguments as
    ``chunk_forward`` (``fg2``: erase is FG2's per-channel rate); ``blocked`` takes the kernel's
    block arrangement of the Gram adjoints, ``fp16`` rounds every matrix operand to fp16 where
    the kernels do.  Returns a dict like ``oracle.recurrence_bwd`` for one (b, h): dq, dk, dv
    [T, d], dlog_decay, derase, dwrite in their inputs' shapes (dwrite None for a shared gate),
    dS0."""
    C = 64
    rnd = _h if fp16 else (lambda a: a)
    q, k, v = (np.asarray(x, np.float64) for x in (q, k, v))
    T, dk = k.shape
    dv = v.shape[1]
    la_in = np.asarray(log_decay, np.float64)
    la = np.broadcast_to(la_in[:, None] if la_in.ndim == 1 else la_in, (T, dk))
    e_in = np.asarray(erase, np.float64)
    if fg2:
        rt = np.sqrt(e_in)
        kap, vt_all = k * rt, v * rt
        e = np.ones((T, dk))
        w = np.ones((T, dv))
    else:
        kap = k
        e = np.broadcast_to(e_in[:, None] if e_in.ndim == 1 else e_in, (T, dk))
        w_in = e_in if write is None else np.asarray(write, np.float64)
        w = np.broadcast_to(w_in[:, None] if w_in.ndim == 1 else w_in, (T, dv))
        vt_all = w * v
    dO = np.zeros((T, dv)) if dO is None else np.asarray(dO, np.float64)
    nck = (T + C - 1) // C

    def pad(x, n):
        return np.concatenate([x, np.zeros((C - n,) + x.shape[1:])]) if n < C else x

    # per-chunk factors, forward
    chunks = []
    S = np.zeros((dk, dv)) if S0 is None else np.array(S0, np.float64)
    for c in range(nck):
        c0 = C * c
        n = min(C, T - c0)
        sl = slice(c0, c0 + n)
        x = dict(k=pad(kap[sl], n), q=pad(q[sl], n), u=pad(e[sl] * kap[sl], n), vt=pad(vt_all[sl], n),
                 la=pad(la[sl], n), dO=pad(dO[sl], n), n=n, sl=sl)
        g = np.cumsum(x["la"], axis=0)
        gC = g[-1]
        Kp, Qp = x["k"] * np.exp(g), x["q"] * np.exp(g)
        Ke, Ue = x["k"] * np.exp(gC - g), x["u"] * np.exp(gC - g)
        Akk = _lower(np.einsum("td,id,tid->ti", x["k"], x["k"], _masked_exp_diff(g, True)), True)
        Aku = _lower(np.einsum("td,id,tid->ti", x["k"], x["u"], _masked_exp_diff(g, True)), True)
        Aqk = _lower(np.einsum("td,id,tid->ti", x["q"], x["k"], _masked_exp_diff(g, False)), False)
        Aqu = _lower(np.einsum("td,id,tid->ti", x["q"], x["u"], _masked_exp_diff(g, False)), False)
        Tm = np.linalg.inv(np.eye(C) + Aku)
        M = Tm @ (Kp @ S + Akk @ x["vt"])
        x.update(g=g, gC=gC, Kp=Kp, Qp=Qp, Ke=Ke, Ue=Ue, Akk=Akk, Aku=Aku, Aqk=Aqk, Aqu=Aqu, Tm=Tm, S=S.copy(),
                 M=M, Delta=x["vt"] - M)
        chunks.append(x)
        S = np.exp(gC)[:, None] * S + Ke.T @ x["vt"] - Ue.T @ M

    # adjoint scan: G at every chunk end, and Z
    G = np.zeros((dk, dv)) if dS_T is None else np.array(dS_T, np.float64)
    for x in reversed(chunks):
        x["G"] = G.copy()
        x["Z"] = -x["Tm"].T @ (x["Aqu"].T @ x["dO"] + x["Ue"] @ G)
        G = np.exp(x["gC"])[:, None] * G + x["Qp"].T @ x["dO"] + x["Kp"].T @ x["Z"]
    dS0 = G

    out = {n: np.zeros((T, d)) for n, d in (("dq", dk), ("dk", dk), ("dv", dv), ("dla", dk), ("de", dk), ("dw", dv))}
    for x in chunks:
        n, sl = x["n"], x["sl"]
        S, G, Z, dOc = rnd(x["S"]), rnd(x["G"]), rnd(x["Z"]), rnd(x["dO"])
        Vt = rnd(x["vt"])
        Mx = rnd(x["Delta"] if fg2 else x["M"])
        # the products with the state and its adjoint
        dKp, dQp = Z @ S.T, dOc @ S.T
        dGam = np.sum(x["S"] * x["G"], axis=1)
        if fg2:
            dKe, dUe = Mx @ G.T, np.zeros((C, dk))
            dAkk, dAku = _lower(Z @ Mx.T, True), np.zeros((C, C))
            dAqk, dAqu = _lower(dOc @ Mx.T, False), np.zeros((C, C))
            dVt = -x["Z"]
        else:
            dKe, dUe = Vt @ G.T, -Mx @ G.T
            dAkk, dAku = _lower(Z @ Vt.T, True), -_lower(Z @ Mx.T, True)
            dAqk, dAqu = _lower(dOc @ Vt.T, False), -_lower(dOc @ Mx.T, False)
            dVt = rnd(x["Akk"]).T @ Z + rnd(x["Aqk"]).T @ dOc + rnd(x["Ke"]) @ G
        # through the Gram matrices
        gb = gram_bwd_blocked if blocked else (lambda dA, a, b, g, s: gram_bwd_exact(dA, a, b, g, s))
        kw = dict(rnd=rnd) if blocked else {}
        g, kk, qq, uu = x["g"], x["k"], x["q"], x["u"]
        r1, c1 = gb(dAkk, kk, kk, g, True, **kw)
        r2, c2 = gb(dAku, kk, uu, g, True, **kw)
        r3, c3 = gb(dAqk, qq, kk, g, False, **kw)
        r4, c4 = gb(dAqu, qq, uu, g, False, **kw)
        k_row, q_row, k_col, u_col = r1 + r2, r3 + r4, c1 + c3, c2 + c4
        eg, egn = np.exp(g), np.exp(x["gC"] - g)
        dkap = eg * dKp + egn * dKe + k_row + k_col
        du = egn * dUe + u_col
        dq = eg * dQp + q_row
        dg = (kk * eg * dKp + qq * eg * dQp - kk * egn * dKe - uu * egn * dUe
              + kk * k_row + qq * q_row - kk * k_col - uu * u_col)
        dg[n - 1] += np.sum(kk * egn * dKe + uu * egn * dUe, axis=0) + np.exp(x["gC"]) * dGam
        dla = np.cumsum(dg[::-1], axis=0)[::-1]
        ec = pad(e[sl], n)
        wc = pad(w[sl], n)
        vc = pad(v[sl], n)
        out["dq"][sl] = dq[:n]
        out["dla"][sl] = dla[:n]
        if fg2:
            out["dk"][sl] = dkap[:n]  # k~'s adjoint; scaled below
            out["dv"][sl] = dVt[:n]
        else:
            out["dk"][sl] = (dkap + ec * du)[:n]
            out["de"][sl] = (kk * du)[:n]
            out["dv"][sl] = (wc * dVt)[:n]
            out["dw"][sl] = (vc * dVt)[:n]
    res = dict(dq=out["dq"], dS0=dS0)
    res["dlog_decay"] = out["dla"].sum(-1) if la_in.ndim == 1 else out["dla"]
    if fg2:
        res["dk"] = rt * out["dk"]
        res["dv"] = rt * out["dv"]
        res["dbeta"] = (k * out["dk"] + v * out["dv"]) / (2 * rt)
        return res
    res["dk"], res["dv"] = out["dk"], out["dv"]
    de = out["de"].sum(-1) if e_in.ndim == 1 else out["de"]
    if write is None:
        dw = out["dw"].sum(-1) if e_in.ndim == 1 else out["dw"]
        res["derase"], res["dwrite"] = de + dw, None
    else:
        w_nd = np.asarray(write).ndim
        res["derase"], res["dwrite"] = de, (out["dw"].sum(-1) if w_nd == 1 else out["dw"])
    return res


# ------------------------------------------------------------------------------------------
# Segment-parallel evaluation (the full-width scan's algebra).  The chunk map is affine in the
# incoming state, S_out = F S_in + H, so a sequence cut into segments of whole chunks can form
# every segment's (F, H) independently -- F from S = I with no values, H from S = 0 -- chain
# S_in[s + 1] = F[s] S_in[s] + H[s], and run every segment from its true entering state
# ("Linearized 2-Simplicial Attention" page, method: states rebuilt from boundary states;
# "FG2-GDN" page, section 3: the chunked structure that per-channel rates keep).
# ------------------------------------------------------------------------------------------
def wide_plan(bh, T, chunk=64):
    """The library's segment plan for B * H = bh heads of T tokens: (segments, first length,
    other length) in chunks -- P - 1 = min(256 / bh, 8), at most half the chunks, the first
    segment 0.7 times as long as the others."""
    nch = -(-T // chunk)
    if nch == 0:
        return 1, 0, 0
    p = 1 if bh >= 256 else 1 + min(256 // bh, 8)
    if p > nch // 2:
        p = nch // 2 if nch // 2 > 1 else 1
    if p <= 1:
        return 1, nch, nch
    L = 10 * nch // (10 * p - 3)
    return p, nch - (p - 1) * L, L


def segmented_forward(q, k, v, log_decay, erase, write=None, S0=None, bounds=None, chunk=64):
    """chunk_forward of one (b, h) evaluated segment by segment.  bounds: the chunk indices where
    segments start (first 0).  Returns (o, S_T, F, H) with F, H of every segment but the last."""
    q, k, v = (np.asarray(x, np.float64) for x in (q, k, v))
    T, dk = k.shape
    nch = -(-T // chunk)
    starts = [b * chunk for b in bounds] + [T]
    sym = np.asarray(erase).ndim == 1 and write is None

    def part(a, s, e):
        return None if a is None else np.asarray(a, np.float64)[s:e]

    o = np.zeros((T, v.shape[1]))
    S_in = np.zeros((dk, v.shape[1])) if S0 is None else np.array(S0, np.float64)
    Fs, Hs = [], []
    for i in range(len(starts) - 1):
        s, e = starts[i], starts[i + 1]
        args = (part(q, s, e), part(k, s, e))
        gates = (part(log_decay, s, e), part(erase, s, e))
        if i < len(starts) - 2:
            # the segment's map: F from S = I without values, H from S = 0
            _, F = chunk_forward(*args, np.zeros((e - s, dk)), *gates, None if write is None else
                                 np.zeros((e - s, dk)), np.eye(dk), chunk, symmetric=sym)
            _, Hm = chunk_forward(*args, part(v, s, e), *gates, part(write, s, e), None, chunk, symmetric=sym)
            Fs.append(F)
            Hs.append(Hm)
        o[s:e], S_out = chunk_forward(*args, part(v, s, e), *gates, part(write, s, e), S_in, chunk, symmetric=sym)
        if i < len(starts) - 2:
            # what the compose step gives the next segment, from the maps alone
            S_in = Fs[-1] @ S_in + Hs[-1]
        else:
            S_in = S_out
    assert nch == 0 or starts[-2] < T
    return o, S_in, Fs, Hs
