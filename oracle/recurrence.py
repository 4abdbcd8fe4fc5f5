"""fp64 CPU oracle for the gated delta-rule recurrence.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path (the HIP library, its C ABI or the
Python binding in ``gated_delta_rule_dr_amd``) imports, links or calls this module; only the
test suite, the smoke check in ``__graft_entry__`` and the ``cpu_baseline`` leg of ``bench.py``
use it.  It shares no code with the GPU path.

What it computes
----------------
Per batch ``b`` and head ``h`` the state is a fixed-size associative memory S (dk x dv) that
replaces a growing key/value cache ("KronLSTM ... delta rule", section "The problem": linear
attention keeps a fixed-size matrix, the delta rule first subtracts what is already associated
with the key and then writes the new value).  One token step, in the general form that covers
every variant on the pages:

    S'  = Diag(a_t) S_{t-1}                      (decay, a_t = exp(log_decay_t))
    S_t = S' - (e_t * k_t) (k_t^T S') + k_t (w_t * v_t)^T
    o_t = S_t^T q_t

* erase gate e_t acts on the key side and write gate w_t on the value side, with the decay
  inherited from KDA ("Gated DeltaNet-2: decoupling erase and write in linear attention",
  section "Gated DeltaNet-2: the solution", gate table; "FG2-GDN", section 2, FG2-GDN+ variant
  with separate erase and write strengths).
* KDA: channel decay vector, one scalar beta used for both erase and write, giving
  S_t = (I - beta k k^T) Diag(a_t) S_{t-1} + beta k v^T ("FG2-GDN", section 1 and section 2
  update rule with a scalar beta).
* scalar-gate Gated DeltaNet: a_t = alpha_t * 1; the scalar commutes with (I - beta k k^T).
* the output reads the state after the token's own write (o_t = S_t^T q_t).

Readings taken where the pages are silent (each is listed with its reason in the design notes):
decay is applied before the erase and the write; the decay is passed in log space and
exponentiated here in fp64 from the stored fp32 value; no query scaling and no key
normalisation happen inside the operation (the caller supplies normalised k); ``write=None``
means the write gate equals the erase gate.

Precision: every input is upcast to fp64 as stored (bf16 or fp32 values), and all arithmetic
is fp64.  The loop is the plain token-by-token definition; it is vectorised only across the
independent (b, h) pairs.
"""
from __future__ import annotations

import numpy as np

__all__ = ["recurrence", "recurrence_bwd", "recurrence_fg2", "recurrence_fg2_bwd", "recurrence_varlen", "decode_step",
           "as_f64"]


def as_f64(x):
    """Return ``x`` as a float64 numpy array (torch tensors are moved to the CPU first)."""
    if x is None:
        return None
    if hasattr(x, "detach"):  # a torch tensor; keep torch optional for the oracle itself
        import torch

        return x.detach().to("cpu", torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def _gate(g, B, T, H, d, name):
    """Broadcast a per-head gate [B,T,H] or per-channel gate [B,T,H,d] to [B,H,T,d|1]."""
    if g.ndim == 3:
        if g.shape != (B, T, H):
            raise ValueError(f"{name}: per-head gate must be [B,T,H], got {g.shape}")
        return np.transpose(g, (0, 2, 1))[..., None]
    if g.ndim == 4:
        if g.shape != (B, T, H, d):
            raise ValueError(f"{name}: per-channel gate must be [B,T,H,{d}], got {g.shape}")
        return np.transpose(g, (0, 2, 1, 3))
    raise ValueError(f"{name}: gate must have 3 or 4 dims, got {g.ndim}")


def recurrence(q, k, v, log_decay, erase, write=None, S0=None, return_states=False):
    """Run the general gated delta-rule recurrence token by token in fp64.

    Args:
      q, k: [B, T, H, dk];  v: [B, T, H, dv]
      log_decay: log a_t <= 0, [B, T, H] (scalar per head) or [B, T, H, dk] (per channel)
      erase: e_t, [B, T, H] or [B, T, H, dk]
      write: w_t, [B, T, H] or [B, T, H, dv]; ``None`` means the write gate is the erase gate
        (then a per-channel erase gate needs dk == dv)
      S0: initial state [B, H, dk, dv] or ``None`` for zeros
      return_states: also return every S_t as [B, H, T, dk, dv] (small cases only)

    Returns:
      (o [B, T, H, dv], S_T [B, H, dk, dv]) as float64, plus the states if requested.
    """
    q, k, v = as_f64(q), as_f64(k), as_f64(v)
    log_decay, erase, write, S0 = as_f64(log_decay), as_f64(erase), as_f64(write), as_f64(S0)
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    if k.shape != (B, T, H, dk) or v.shape[:3] != (B, T, H):
        raise ValueError("q, k, v shapes disagree")
    if write is None:
        write = erase
        if write.ndim == 4 and dk != dv:
            raise ValueError("write=None with a per-channel erase gate needs dk == dv")

    a = np.exp(_gate(log_decay, B, T, H, dk, "log_decay"))  # [B,H,T,dk|1]
    e = _gate(erase, B, T, H, dk, "erase")
    w = _gate(write, B, T, H, dv, "write")
    qh = np.transpose(q, (0, 2, 1, 3))  # [B,H,T,dk]
    kh = np.transpose(k, (0, 2, 1, 3))
    vh = np.transpose(v, (0, 2, 1, 3))

    S = np.zeros((B, H, dk, dv)) if S0 is None else np.array(S0, dtype=np.float64, copy=True)
    if S.shape != (B, H, dk, dv):
        raise ValueError(f"S0 must be [B,H,dk,dv]={B, H, dk, dv}, got {S.shape}")
    o = np.empty((B, H, T, dv))
    states = np.empty((B, H, T, dk, dv)) if return_states else None

    for t in range(T):
        kt = kh[:, :, t, :]  # [B,H,dk]
        S = a[:, :, t, :][..., :, None] * S  # S' = Diag(a_t) S_{t-1}
        m = np.matmul(kt[..., None, :], S)[..., 0, :]  # k_t^T S'        [B,H,dv]
        u = e[:, :, t, :] * kt  # erase acts on the key side   [B,H,dk]
        vw = w[:, :, t, :] * vh[:, :, t, :]  # write acts on the value side [B,H,dv]
        S = S - u[..., :, None] * m[..., None, :] + kt[..., :, None] * vw[..., None, :]
        o[:, :, t, :] = np.matmul(qh[:, :, t, :][..., None, :], S)[..., 0, :]  # S_t^T q_t
        if return_states:
            states[:, :, t] = S

    o = np.transpose(o, (0, 2, 1, 3))
    if return_states:
        return o, S, states
    return o, S


def recurrence_bwd(q, k, v, log_decay, erase, write=None, S0=None, dO=None, dS_T=None):
    """Gradients of the recurrence, by the adjoint of the token loop, in fp64.

    The forward pass of training is the recurrence itself (the chunked form is how it is
    evaluated fast, "FG2-GDN ...", sections 2-3: chunk-parallel training through the WY form);
    its gradients are those of the scalar objective L = sum(o * dO) + sum(S_T * dS_T).  Walking
    the tokens backwards with the state's adjoint G = dL/dS_t (starting from dS_T), one token
    t of the forward step

        S' = Diag(a) S_{t-1},  m = S'^T k,  u = e * k,  v~ = w * v,
        S_t = S' - u m^T + k v~^T,  o_t = S_t^T q_t

    contributes, in reverse order:
        G    += q dO_t^T                       dq_t = S_t dO_t
        dm    = -G^T u                         du   = -G m          dv~ = G^T k
        dk_t  = G v~ + S' dm + e * du          de_t = k * du        (summed over channels
        dw_t  = v * dv~                        dv_t = w * dv~        for a per-head gate)
        G'    = G + k dm^T                     d(log a_t) = a * rowsum(G' * S_{t-1})
        G     = Diag(a) G'                     (the adjoint of S_{t-1});  dS0 = G at the end.
    With ``write=None`` the gate is shared, so its gradient is de + dw.

    Args: as ``recurrence``, plus dO [B, T, H, dv] and dS_T [B, H, dk, dv] (None: zero).
    Returns a dict of float64 arrays: dq, dk, dv, dlog_decay, derase, dwrite (None when
    ``write`` is None), dS0, each shaped like its input (dS0 like S0, or [B, H, dk, dv]).
    """
    q, k, v = as_f64(q), as_f64(k), as_f64(v)
    log_decay, erase, write, S0 = as_f64(log_decay), as_f64(erase), as_f64(write), as_f64(S0)
    dO, dS_T = as_f64(dO), as_f64(dS_T)
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    shared = write is None
    if shared:
        write = erase
        if write.ndim == 4 and dk != dv:
            raise ValueError("write=None with a per-channel erase gate needs dk == dv")
    a = np.exp(_gate(log_decay, B, T, H, dk, "log_decay"))  # [B,H,T,dk|1]
    e = _gate(erase, B, T, H, dk, "erase")
    w = _gate(write, B, T, H, dv, "write")
    qh, kh, vh = (np.transpose(x, (0, 2, 1, 3)) for x in (q, k, v))
    dOh = np.transpose(dO, (0, 2, 1, 3))

    # forward, keeping S_{t-1} of every token
    S = np.zeros((B, H, dk, dv)) if S0 is None else np.array(S0, dtype=np.float64, copy=True)
    prev = np.empty((T, B, H, dk, dv))
    for t in range(T):
        prev[t] = S
        kt = kh[:, :, t]
        Sp = a[:, :, t][..., :, None] * S
        m = np.einsum("bhi,bhij->bhj", kt, Sp)
        S = Sp - (e[:, :, t] * kt)[..., :, None] * m[..., None, :] + kt[..., :, None] * (w[:, :, t] * vh[:, :, t])[..., None, :]

    G = np.zeros((B, H, dk, dv)) if dS_T is None else np.array(dS_T, dtype=np.float64, copy=True)
    gq, gk, gv = np.zeros_like(qh), np.zeros_like(kh), np.zeros_like(vh)
    ga = np.zeros(a.shape[:3] + (dk,))
    ge = np.zeros(e.shape[:3] + (dk,))
    gw = np.zeros(w.shape[:3] + (dv,))
    for t in reversed(range(T)):
        kt, qt, vt, dot = kh[:, :, t], qh[:, :, t], vh[:, :, t], dOh[:, :, t]
        at = a[:, :, t] * np.ones(dk)
        et = e[:, :, t] * np.ones(dk)
        wt = w[:, :, t] * np.ones(dv)
        Sm1 = prev[t]
        Sp = at[..., :, None] * Sm1
        m = np.einsum("bhi,bhij->bhj", kt, Sp)
        u = et * kt
        vw = wt * vt
        St = Sp - u[..., :, None] * m[..., None, :] + kt[..., :, None] * vw[..., None, :]
        G = G + qt[..., :, None] * dot[..., None, :]
        gq[:, :, t] = np.einsum("bhij,bhj->bhi", St, dot)
        dm = -np.einsum("bhij,bhi->bhj", G, u)
        du = -np.einsum("bhij,bhj->bhi", G, m)
        dvw = np.einsum("bhij,bhi->bhj", G, kt)
        gk[:, :, t] = np.einsum("bhij,bhj->bhi", G, vw) + np.einsum("bhij,bhj->bhi", Sp, dm) + et * du
        ge[:, :, t] = kt * du
        gw[:, :, t] = vt * dvw
        gv[:, :, t] = wt * dvw
        Gp = G + kt[..., :, None] * dm[..., None, :]
        ga[:, :, t] = at * np.sum(Gp * Sm1, axis=-1)
        G = at[..., :, None] * Gp

    def back(x, like):  # [B,H,T,d] -> the input's layout, summed over channels for a per-head gate
        x = np.transpose(x, (0, 2, 1, 3))
        return x.sum(-1) if like.ndim == 3 else x

    out = dict(dq=np.transpose(gq, (0, 2, 1, 3)), dk=np.transpose(gk, (0, 2, 1, 3)),
               dv=np.transpose(gv, (0, 2, 1, 3)), dlog_decay=back(ga, log_decay), dS0=G)
    de, dw = back(ge, erase), back(gw, write)
    if shared:
        out["derase"], out["dwrite"] = de + dw, None
    else:
        out["derase"], out["dwrite"] = de, dw
    return out


def recurrence_fg2(q, k, v, log_decay, beta, S0=None):
    """FG2-GDN's update with a per-channel learning rate, token by token in fp64.

    The rate beta_t in R^dk is absorbed symmetrically into the key and the value, which keeps
    the rank-1 Householder form of the update ("FG2-GDN: Enhancing Long-Context Gated Delta
    Networks with Doubly Fine-Grained Control", section 2, FG2-GDN update rule):

        k~_t = sqrt(beta_t) * k_t,   v~_t = sqrt(beta_t) * v_t
        S_t  = (I - k~_t k~_t^T) Diag(a_t) S_{t-1} + k~_t v~_t^T,      o_t = S_t^T q_t

    The rate multiplies value channels, so it needs dk == dv.  The query is not scaled (the
    update rule scales only k and v).  With the scaled pair this is the general recurrence with
    unit erase and write gates, which is how it is evaluated here.

    Args: q, k, v [B, T, H, d]; log_decay [B, T, H] or [B, T, H, d]; beta [B, T, H, d] > 0;
    S0 [B, H, d, d] or None.  Returns (o [B, T, H, d], S_T [B, H, d, d]) as float64.
    """
    q, k, v = as_f64(q), as_f64(k), as_f64(v)
    beta = as_f64(beta)
    if k.shape[-1] != v.shape[-1] or beta.shape != k.shape:
        raise ValueError("the per-channel rate needs dk == dv and beta shaped like k")
    r = np.sqrt(beta)
    ones = np.ones(k.shape[:3])
    return recurrence(q, r * k, r * v, log_decay, ones, None, S0)


def recurrence_fg2_bwd(q, k, v, log_decay, beta, S0=None, dO=None, dS_T=None):
    """Gradients of FG2-GDN's rate form (``recurrence_fg2``), in fp64: the adjoint of the
    recurrence on the scaled pair (k~, v~) = (sqrt(beta) k, sqrt(beta) v) with unit gates, then
    the chain rule through the scaling: dk = sqrt(beta) dk~, dv = sqrt(beta) dv~ and
    dbeta = (k dk~ + v dv~) / (2 sqrt(beta)).  Returns dq, dk, dv, dlog_decay, dbeta, dS0."""
    q, k, v, beta = as_f64(q), as_f64(k), as_f64(v), as_f64(beta)
    r = np.sqrt(beta)
    g = recurrence_bwd(q, r * k, r * v, log_decay, np.ones(k.shape[:3]), None, S0, dO, dS_T)
    return dict(dq=g["dq"], dk=r * g["dk"], dv=r * g["dv"], dlog_decay=g["dlog_decay"],
                dbeta=(k * g["dk"] + v * g["dv"]) / (2 * r), dS0=g["dS0"])


def decode_step(q, k, v, log_decay, erase, write, S):
    """One token of the recurrence for a batch of independent sequences.

    Args use the single-token layout [N, H, d] (gates [N, H] or [N, H, d]); S is [N, H, dk, dv].
    Returns (o [N, H, dv], S_new [N, H, dk, dv]) in fp64; the input state is not modified.
    """
    q, k, v = as_f64(q), as_f64(k), as_f64(v)
    log_decay, erase, write = as_f64(log_decay), as_f64(erase), as_f64(write)

    def tok(x):
        return None if x is None else x[:, None]

    o, S_new = recurrence(tok(q), tok(k), tok(v), tok(log_decay), tok(erase), tok(write), S)
    return o[:, 0], S_new


def recurrence_varlen(q, k, v, log_decay, erase, write=None, S0=None, cu_seqlens=None):
    """The recurrence over a packed batch of independent sequences of different lengths.

    Each sequence keeps its own fixed-size state, started from its own initial state, and no
    state crosses from one sequence to the next: linear attention replaces the growing cache
    of each sequence by one fixed-size memory, which is what lets a server hold one state per
    conversation and decode it in constant memory ("Gated DeltaNet-2: decoupling erase and
    write in linear attention", sections "The attention bottleneck" and "Why this matters";
    "KronLSTM ...", section "The problem").  Packing the sequences one after another on the
    token axis, delimited by offsets, is a layout convention that those sections do not describe.

    Args:
      q, k: [1, T, H, dk] and v: [1, T, H, dv], the sequences concatenated on the token axis;
        gates [1, T, H] or [1, T, H, d] likewise (``write=None``: the erase gate).
      cu_seqlens: N + 1 offsets, cu_seqlens[0] == 0, nondecreasing, cu_seqlens[N] == T;
        sequence n holds tokens cu_seqlens[n] .. cu_seqlens[n + 1] - 1 (it may be empty).
      S0: [N, H, dk, dv] initial states, or ``None`` for zeros.

    Returns:
      (o [1, T, H, dv], S_T [N, H, dk, dv]) as float64; an empty sequence has S_T[n] = S0[n].
    """
    q, k, v = as_f64(q), as_f64(k), as_f64(v)
    log_decay, erase, write, S0 = as_f64(log_decay), as_f64(erase), as_f64(write), as_f64(S0)
    cu = np.asarray(cu_seqlens if not hasattr(cu_seqlens, "detach") else cu_seqlens.cpu().numpy())
    cu = cu.astype(np.int64)
    if q.ndim != 4 or q.shape[0] != 1:
        raise ValueError("packed inputs have a leading batch dimension of 1")
    _, T, H, dk = q.shape
    dv = v.shape[-1]
    N = len(cu) - 1
    if N < 0 or cu[0] != 0 or cu[-1] != T or np.any(np.diff(cu) < 0):
        raise ValueError("cu_seqlens must start at 0, end at T and never decrease")
    if S0 is not None and S0.shape != (N, H, dk, dv):
        raise ValueError(f"S0 must be [N,H,dk,dv]={N, H, dk, dv}, got {S0.shape}")

    def part(x, lo, hi):
        return None if x is None else x[:, lo:hi]

    o = np.zeros((1, T, H, dv))
    S_T = np.empty((N, H, dk, dv))
    for n in range(N):
        lo, hi = int(cu[n]), int(cu[n + 1])
        s0 = None if S0 is None else S0[n : n + 1]
        if hi == lo:
            S_T[n] = 0.0 if S0 is None else S0[n]
            continue
        o_n, S_n = recurrence(part(q, lo, hi), part(k, lo, hi), part(v, lo, hi),
                              part(log_decay, lo, hi), part(erase, lo, hi), part(write, lo, hi), s0)
        o[:, lo:hi] = o_n
        S_T[n] = S_n[0]
    return o, S_T
