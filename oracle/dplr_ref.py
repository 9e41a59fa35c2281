"""CPU oracle for the general diagonal-plus-low-rank (DPLR) recurrence that KDA
is a restricted case of.  TEST INFRASTRUCTURE: only the test suite and the
benchmark's parity and baseline legs may import this module.  It shares no
code with the GPU library.

Page "Kimi K3论文：Kimi Linear", section 4: the general gated delta rule has a
diagonal-plus-low-rank transition,

    S_t = (D_t - a_t b_t^T) S_{t-1} + k_t v_t^T,        o_t = S_t^T q_t,

with D_t = Diag(alpha_t) and a_t, b_t free vectors; KDA is the case
a_t = beta_t k_t, b_t = k_t * alpha_t (and the write beta_t k_t v_t^T).  The
page gives no output rule for DPLR; o_t = S_t^T q_t is taken from KDA's
(section 3), and the gate is passed in log space, g_t = log(alpha_t), as for
KDA.

:func:`recurrent` is that recurrence, one token at a time, in fp64.
:func:`chunked` is the chunkwise reorganisation the GPU kernels follow (not
printed on the pages; derived below and checked against :func:`recurrent`).
For a chunk with entry state S, G = in-chunk cumulative sum of g (G_0 = 0),
and u_i = S_{i-1}^T b_i (what the low-rank term reads before step i):

    S_r = Diag(e^{G_r}) S + sum_{i<=r} Diag(e^{G_r - G_i}) (k_i v_i^T - a_i u_i^T)

so u_i depends on S and on the u_j, j < i:

    Bh  = e^{G_{r-1}} * b,   Qh = e^{G_r} * q,   Kb = e^{-G} * k,   Ab = e^{-G} * a
    A_qk = tril(Qh Kb^T),  A_qa = tril(Qh Ab^T),                  (i <= r)
    A_bk = stril(Bh Kb^T), A_ba = stril(Bh Ab^T)                   (i < r)
    U   = (I + A_ba)^{-1} (Bh S + A_bk V)
    O   = Qh S + A_qk V - A_qa U
    S  <- Diag(e^{G_L}) (S + Kb^T V - Ab^T U)

Four intra-chunk matrices where KDA needs two (Aqk and Akk), which is the
difference the page's section 4 points to.  Here every decay difference is
exponentiated directly in fp64 (no factorisation).
"""
from __future__ import annotations

import numpy as np

from oracle.kda_ref import forward_substitution


def _f64(x):
    if x is None:
        return None
    if hasattr(x, "detach"):
        x = x.detach().to("cpu").double().numpy()
    return np.asarray(x, dtype=np.float64)


def recurrent_head(q, k, v, a, b, g, S0=None):
    """One head: q, k, a, b, g [T, dk], v [T, dv], S0 [dk, dv] or None.
    Returns (o [T, dv], S_T [dk, dv]) in fp64."""
    q, k, v, a, b, g = (_f64(x) for x in (q, k, v, a, b, g))
    T, dk = q.shape
    S = np.zeros((dk, v.shape[1])) if S0 is None else _f64(S0).copy()
    o = np.zeros((T, v.shape[1]))
    for t in range(T):
        u = S.T @ b[t]                                   # read of the low-rank term
        S = np.exp(g[t])[:, None] * S - np.outer(a[t], u) + np.outer(k[t], v[t])
        o[t] = S.T @ q[t]
    return o, S


def recurrent(q, k, v, a, b, g, S0=None, heads=None):
    """[B, T, H, d] inputs (S0 [B, H, dk, dv] or None).  Returns o [B, T, H', dv]
    and S_T [B, H', dk, dv] in fp64 for the (b, h) pairs in ``heads`` (default:
    all, in order)."""
    B, T, H, _ = q.shape
    pairs = [(bb, hh) for bb in range(B) for hh in range(H)] if heads is None else list(heads)
    dv = v.shape[-1]
    if heads is None:
        o = np.zeros((B, T, H, dv))
        S = np.zeros((B, H, q.shape[-1], dv))
    else:
        o = np.zeros((len(pairs), T, dv))
        S = np.zeros((len(pairs), q.shape[-1], dv))
    for n, (bb, hh) in enumerate(pairs):
        s0 = None if S0 is None else S0[bb, hh]
        oh, sh = recurrent_head(q[bb, :, hh], k[bb, :, hh], v[bb, :, hh], a[bb, :, hh], b[bb, :, hh],
                                g[bb, :, hh], s0)
        if heads is None:
            o[bb, :, hh], S[bb, hh] = oh, sh
        else:
            o[n], S[n] = oh, sh
    return o, S


def chunked_head(q, k, v, a, b, g, S0=None, C: int = 64):
    """The chunkwise form of the module docstring for one head (the last chunk
    may be shorter)."""
    q, k, v, a, b, g = (_f64(x) for x in (q, k, v, a, b, g))
    T, dk = q.shape
    dv = v.shape[1]
    S = np.zeros((dk, dv)) if S0 is None else _f64(S0).copy()
    o = np.zeros((T, dv))
    for s in range(0, T, C):
        e = min(s + C, T)
        Q, K, V, A, Bv, Gs = q[s:e], k[s:e], v[s:e], a[s:e], b[s:e], g[s:e]
        L = e - s
        G = np.cumsum(Gs, axis=0)
        Gprev = G - Gs                                   # G_{r-1}, zero for the first row
        Dqk = np.exp(G[:, None, :] - G[None, :, :])      # e^{G_r - G_i}      [r, i, c]
        Dbk = np.exp(Gprev[:, None, :] - G[None, :, :])  # e^{G_{r-1} - G_i}  [r, i, c]
        A_qk = np.tril(np.einsum("rc,ic,ric->ri", Q, K, Dqk), 0)
        A_qa = np.tril(np.einsum("rc,ic,ric->ri", Q, A, Dqk), 0)
        A_bk = np.tril(np.einsum("rc,ic,ric->ri", Bv, K, Dbk), -1)
        A_ba = np.tril(np.einsum("rc,ic,ric->ri", Bv, A, Dbk), -1)
        Tm = forward_substitution(A_ba)                  # (I + A_ba)^{-1}
        U = Tm @ ((np.exp(Gprev) * Bv) @ S + A_bk @ V)
        o[s:e] = (np.exp(G) * Q) @ S + A_qk @ V - A_qa @ U
        GL = G[L - 1]
        Kt = np.exp(GL[None, :] - G)                     # e^{G_L - G_i}
        S = np.exp(GL)[:, None] * S + (Kt * K).T @ V - (Kt * A).T @ U
    return o, S
