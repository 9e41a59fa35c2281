"""CPU oracle for Kimi Delta Attention (KDA).  TEST INFRASTRUCTURE.

Only the test suite, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this module.  It shares no code with the GPU library and
imports nothing from it.

Contents (all fp64):

* :func:`recurrent` -- the oracle proper: the sequential recurrence of eq. (1) on
  page "Kimi K3论文：Kimi Linear" (section 3), in plain C (``kda_ref.c``),
  loaded through ctypes.
* :func:`recurrent_grad` -- the gradient oracle: reverse mode through the same
  recurrence, in plain C, for the backward pass of the chunked form (dq, dk,
  dv, d log(alpha), d beta, dS0 from dL/do and dL/dS_T).
* Independent cross-forms that the tests use to pin the oracle.  Each follows a
  different passage, so a dropped term, a wrong sign or a swapped gate order in
  one of them shows up as a mismatch:

  - :func:`dplr_form` -- the diagonal-plus-low-rank rewrite of eq. (1),
    page "Kimi K3论文：Kimi Linear", section 4.
  - :func:`chunked_form` -- the chunkwise algorithm: in-chunk cumulative decay,
    the two masked intra-chunk matrices, forward substitution for the inverse of
    the unit-lower-triangular matrix, WY factors and the chunk-to-chunk state
    pass.  Page "Kimi Linear：高效注意力机制在长序列处理中的创新应用",
    sections 2.1-2.3; page "Kimi K3论文：Kimi Linear", section 4.
  - :func:`proposition_states` -- the Proposition S_r = P_r S_0 + H_r with the
    auxiliary vectors w_r, u_r, written out per token (page "Kimi Linear：
    高效注意力机制在长序列处理中的创新应用", sections 2.1-2.2).
  - :func:`product_form` -- the transition-product form used to argue that
    KDA acts as a learnable position encoding (page "Kimi K3论文：Kimi Linear",
    section 6), with the write strength beta_i and the gate order of eq. (1).
  - :func:`autograd_grad` -- torch autograd (CPU, fp64) through a torch
    transcription of the recurrence, against which :func:`recurrent_grad` is
    checked (besides central finite differences of :func:`recurrent`).
  - :func:`deltanet`, :func:`gated_deltanet` -- the two predecessors of KDA
    (page "Kimi K3论文：Kimi Linear", section 2), which KDA must reduce to.

Readings of points the pages leave open are listed where they are used.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import sysconfig

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kda_ref.c")
_LIB_PATH = os.path.join(_HERE, "libkda_ref.so")
_lib = None


def build(force: bool = False) -> str:
    """Compile ``kda_ref.c`` into ``libkda_ref.so`` with gcc -O2 -fopenmp."""
    if force or not os.path.exists(_LIB_PATH) or (
        os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC)
    ):
        tmp = _LIB_PATH + ".tmp"
        cmd = ["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-std=c99",
               "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        build()
        lib = ctypes.CDLL(_LIB_PATH)
        dp = ctypes.POINTER(ctypes.c_double)
        lib.kda_ref_recurrent.argtypes = [dp, dp, dp, dp, dp, dp, dp, dp,
                                          ctypes.c_long, ctypes.c_long, ctypes.c_long,
                                          ctypes.c_long, ctypes.c_long, ctypes.c_int]
        lib.kda_ref_recurrent.restype = ctypes.c_int
        lib.kda_ref_recurrent_grad.argtypes = [dp] * 14 + [ctypes.c_long] * 5 + [ctypes.c_int]
        lib.kda_ref_recurrent_grad.restype = ctypes.c_int
        lib.kda_ref_max_threads.argtypes = []
        lib.kda_ref_max_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def max_threads() -> int:
    return int(_load().kda_ref_max_threads())


def _f64(x):
    """fp64, C-contiguous copy of an array-like (torch tensors included)."""
    if x is None:
        return None
    if hasattr(x, "detach"):  # torch tensor: upcast exactly (bf16/fp32 -> fp64)
        x = x.detach().to("cpu").double().numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a):
    if a is None:
        return ctypes.POINTER(ctypes.c_double)()
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def recurrent(q, k, v, g, beta, S0=None, nthreads: int = 0):
    """The oracle: eq. (1) of page "Kimi K3论文：Kimi Linear", section 3.

    Shapes: q, k, g ``[B, T, H, dk]``; v ``[B, T, H, dv]``; beta ``[B, T, H]``;
    S0 ``[B, H, dk, dv]`` or None (zeros).  ``g`` is log(alpha).  Inputs of any
    float dtype are upcast exactly to fp64.  Returns ``(o [B,T,H,dv], S_T
    [B,H,dk,dv])`` in fp64.
    """
    q, k, v, g, beta, S0 = (_f64(x) for x in (q, k, v, g, beta, S0))
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    assert k.shape == q.shape and g.shape == q.shape
    assert v.shape == (B, T, H, dv) and beta.shape == (B, T, H)
    if S0 is not None:
        assert S0.shape == (B, H, dk, dv)
    o = np.zeros((B, T, H, dv))
    S_T = np.zeros((B, H, dk, dv))
    rc = _load().kda_ref_recurrent(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                   _ptr(S0), _ptr(o), _ptr(S_T),
                                   B, T, H, dk, dv, int(nthreads))
    if rc != 0:
        raise RuntimeError("kda_ref_recurrent failed")
    return o, S_T


def recurrent_grad(q, k, v, g, beta, S0, dO, dS_T=None, nthreads: int = 0):
    """Gradient oracle: reverse mode through the recurrence of :func:`recurrent`.

    For the scalar loss L = sum(dO * o) + sum(dS_T * S_T) (dS_T None => 0),
    returns ``(dq, dk, dv, dg, dbeta, dS0)`` in fp64 with the shapes of
    q, k, v, g, beta and S0 (dS0 is returned even when S0 is None: it is the
    gradient at the zero state).  The chain rule is taken step by step back
    through eq. (1) of page "Kimi K3论文：Kimi Linear", section 3, in plain C
    (``kda_ref.c``); ``g`` is log(alpha), so dg is the gradient in log space.
    """
    q, k, v, g, beta, S0, dO, dS_T = (_f64(x) for x in (q, k, v, g, beta, S0, dO, dS_T))
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    assert k.shape == q.shape and g.shape == q.shape
    assert v.shape == (B, T, H, dv) and beta.shape == (B, T, H) and dO.shape == v.shape
    for x in (S0, dS_T):
        if x is not None:
            assert x.shape == (B, H, dk, dv)
    out = [np.zeros(x.shape) for x in (q, k, v, g, beta)] + [np.zeros((B, H, dk, dv))]
    rc = _load().kda_ref_recurrent_grad(
        _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(S0), _ptr(dO), _ptr(dS_T),
        *(_ptr(x) for x in out), B, T, H, dk, dv, int(nthreads))
    if rc != 0:
        raise RuntimeError("kda_ref_recurrent_grad failed")
    return tuple(out)


def autograd_grad(q, k, v, g, beta, S0, dO, dS_T=None):
    """Cross-form of :func:`recurrent_grad`: torch autograd (CPU, fp64) through
    the same recurrence written with torch tensor operations, single head:
    q, k, g [T, dk]; v, dO [T, dv]; beta [T]; S0, dS_T [dk, dv] or None."""
    import torch

    def t64(x, req):
        x = torch.zeros(0) if x is None else torch.as_tensor(np.asarray(x, np.float64))
        return x.clone().requires_grad_(req)

    q_, k_, v_, g_, b_ = (t64(x, True) for x in (q, k, v, g, beta))
    dk, dv = q_.shape[1], v_.shape[1]
    S0_ = (torch.zeros(dk, dv, dtype=torch.float64) if S0 is None else t64(S0, False)).clone()
    S0_.requires_grad_(True)
    S = S0_
    outs = []
    for t in range(q_.shape[0]):
        Sp = torch.exp(g_[t])[:, None] * S
        u = b_[t] * (v_[t] - Sp.T @ k_[t])
        S = Sp + torch.outer(k_[t], u)
        outs.append(S.T @ q_[t])
    o = torch.stack(outs) if outs else torch.zeros(0, dv, dtype=torch.float64)
    loss = (o * torch.as_tensor(np.asarray(dO, np.float64))).sum()
    if dS_T is not None:
        loss = loss + (S * torch.as_tensor(np.asarray(dS_T, np.float64))).sum()
    grads = torch.autograd.grad(loss, [q_, k_, v_, g_, b_, S0_], allow_unused=True)
    ref = (q_, k_, v_, g_, b_, S0_)
    return tuple((torch.zeros_like(x) if gr is None else gr).detach().numpy()
                 for gr, x in zip(grads, ref))


# ---------------------------------------------------------------------------
# Cross-forms (numpy, fp64).  Single head: q, k, g [T, dk]; v [T, dv]; beta [T];
# S0 [dk, dv].  ``per_head`` lifts them to the [B, T, H, .] layout.
# ---------------------------------------------------------------------------

def per_head(fn, q, k, v, g, beta, S0=None, **kw):
    """Apply a single-head form to every (b, h) of ``[B, T, H, .]`` inputs."""
    q, k, v, g, beta, S0 = (_f64(x) for x in (q, k, v, g, beta, S0))
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    o = np.zeros((B, T, H, dv))
    S = np.zeros((B, H, dk, dv))
    for b in range(B):
        for h in range(H):
            s0 = None if S0 is None else S0[b, h]
            o[b, :, h], S[b, h] = fn(q[b, :, h], k[b, :, h], v[b, :, h],
                                     g[b, :, h], beta[b, :, h], s0, **kw)
    return o, S


def dplr_form(q, k, v, g, beta, S0=None):
    """Diagonal-plus-low-rank rewrite of eq. (1) (page "Kimi K3论文：Kimi Linear",
    section 4): S_t = (D - a_t b_t^T) S_{t-1} + beta_t k_t v_t^T with
    D = Diag(alpha_t), a_t = beta_t k_t, b_t = k_t * alpha_t.  The full d_k x d_k
    transition matrix is formed explicitly every step."""
    q, k, v, g, beta = (np.asarray(x, np.float64) for x in (q, k, v, g, beta))
    T, dk = q.shape
    dv = v.shape[1]
    S = np.zeros((dk, dv)) if S0 is None else np.array(S0, np.float64)
    o = np.zeros((T, dv))
    for t in range(T):
        alpha = np.exp(g[t])
        a = beta[t] * k[t]
        b = k[t] * alpha
        transition = np.diag(alpha) - np.outer(a, b)
        S = transition @ S + beta[t] * np.outer(k[t], v[t])
        o[t] = S.T @ q[t]
    return o, S


def forward_substitution(A_strict):
    """Inverse of the unit-lower-triangular I + A by forward substitution.

    Follows the loop printed on page "Kimi Linear：高效注意力机制在长序列处理中的
    创新应用", section 2.3 (reading: the matrix it starts from is the negated,
    STRICTLY lower-triangular Akk, and the identity is added after the loop;
    the mask shown on that page keeps the diagonal, which is the mask of Aqk).
    Row i is finished using the original row i and the finished rows j < i.
    """
    N = -np.tril(np.asarray(A_strict, np.float64), -1)
    C = N.shape[0]
    for i in range(1, C):
        N[i, :i] = N[i, :i] + (N[i, :, None] * N[:, :i]).sum(0)
    return N + np.eye(C)


def chunked_form(q, k, v, g, beta, S0=None, C: int = 64):
    """Chunkwise algorithm (page "Kimi Linear：高效注意力机制在长序列处理中的创新
    应用", sections 2.1-2.3; page "Kimi K3论文：Kimi Linear", section 4).

    For each chunk of C tokens (the last one may be shorter) with entry state S:
      G   = in-chunk cumulative sum of g                       (L x dk)
      Akk[r,i] = beta_r sum_c k_r[c] k_i[c] e^{G_r[c]-G_i[c]}, i < r (strict)
      Aqk[r,i] =        sum_c q_r[c] k_i[c] e^{G_r[c]-G_i[c]}, i <= r
      Tm  = (I + Akk)^{-1}                   (forward substitution)
      W   = Tm (beta * e^G * K),   U = Tm (beta * V)           (WY factors)
      Vn  = U - W S
      O   = (e^G * Q) S + Aqk Vn
      S   = Diag(e^{G_L}) S + (e^{G_L - G} * K)^T Vn
    The last four lines are not printed on the pages; they follow from the
    Proposition (see :func:`proposition_states`) by induction.  Here the decay
    differences are exponentiated directly in fp64 (no factorisation).
    """
    q, k, v, g, beta = (np.asarray(x, np.float64) for x in (q, k, v, g, beta))
    T, dk = q.shape
    dv = v.shape[1]
    S = np.zeros((dk, dv)) if S0 is None else np.array(S0, np.float64)
    o = np.zeros((T, dv))
    for s in range(0, T, C):
        e = min(s + C, T)
        Q, K, V, Gs, bt = q[s:e], k[s:e], v[s:e], g[s:e], beta[s:e]
        L = e - s
        G = np.cumsum(Gs, axis=0)
        D = np.exp(G[:, None, :] - G[None, :, :])            # [r, i, c]
        kk = np.einsum("rc,ic,ric->ri", K, K, D)
        qk = np.einsum("rc,ic,ric->ri", Q, K, D)
        Akk = bt[:, None] * np.tril(kk, -1)
        Aqk = np.tril(qk, 0)
        Tm = forward_substitution(Akk)
        W = Tm @ (bt[:, None] * np.exp(G) * K)
        U = Tm @ (bt[:, None] * V)
        Vn = U - W @ S
        o[s:e] = (np.exp(G) * Q) @ S + Aqk @ Vn
        GL = G[L - 1]
        S = np.exp(GL)[:, None] * S + (np.exp(GL[None, :] - G) * K).T @ Vn
    return o, S


def proposition_states(q, k, v, g, beta, S0=None):
    """Per-token states of ONE chunk from the Proposition (page "Kimi Linear：
    高效注意力机制在长序列处理中的创新应用", section 2.1):

        S_r = P_r S_0 + H_r,
        P_r = Diag(gamma_r) - sum_{i<=r} Diag(gamma_{i->r}) k_i w_i^T,
        H_r =                 sum_{i<=r} Diag(gamma_{i->r}) k_i u_i^T,

    reading the run-together formulas with sums over i = 1..r, gamma_{r->r} = 1,
    gamma_r = exp(G_r), gamma_{i->r} = exp(G_r - G_i).  The auxiliary vectors
    (section 2.2, WY representation) come from the recursion
        w_r = beta_r gamma_r * k_r - sum_{i<r} A[r,i] w_i,
        u_r = beta_r v_r           - sum_{i<r} A[r,i] u_i,
        A[r,i] = beta_r sum_c k_r[c] k_i[c] gamma_{i->r}[c].
    Returns (o [L, dv], states [L, dk, dv]).
    """
    q, k, v, g, beta = (np.asarray(x, np.float64) for x in (q, k, v, g, beta))
    L, dk = q.shape
    dv = v.shape[1]
    S0 = np.zeros((dk, dv)) if S0 is None else np.asarray(S0, np.float64)
    G = np.cumsum(g, axis=0)
    w = np.zeros((L, dk))
    u = np.zeros((L, dv))
    for r in range(L):
        w[r] = beta[r] * np.exp(G[r]) * k[r]
        u[r] = beta[r] * v[r]
        for i in range(r):
            a = beta[r] * np.sum(k[r] * k[i] * np.exp(G[r] - G[i]))
            w[r] -= a * w[i]
            u[r] -= a * u[i]
    states = np.zeros((L, dk, dv))
    o = np.zeros((L, dv))
    for r in range(L):
        P = np.diag(np.exp(G[r]))
        Hm = np.zeros((dk, dv))
        for i in range(r + 1):
            dec = np.exp(G[r] - G[i])
            P = P - np.outer(dec * k[i], w[i])
            Hm = Hm + np.outer(dec * k[i], u[i])
        states[r] = P @ S0 + Hm
        o[r] = states[r].T @ q[r]
    return o, states


def product_form(q, k, v, g, beta, S0=None):
    """Transition-product form (page "Kimi K3论文：Kimi Linear", section 6):

        o_t^T = sum_{i<=t} beta_i q_t^T [prod_{j=i+1..t} M_j] k_i v_i^T
                + q_t^T [prod_{j=1..t} M_j] S_0,
        M_j = (I - beta_j k_j k_j^T) Diag(alpha_j),

    products ordered with the latest j on the left.  Reading: the page's
    formula omits beta_i and writes the gate on the other side of the
    Householder factor; the gate order here is that of eq. (1), which the
    rewrite in section 4 confirms.  Brute force, O(T^2 dk^3): tiny inputs only.
    """
    q, k, v, g, beta = (np.asarray(x, np.float64) for x in (q, k, v, g, beta))
    T, dk = q.shape
    dv = v.shape[1]
    S0 = np.zeros((dk, dv)) if S0 is None else np.asarray(S0, np.float64)
    M = [(np.eye(dk) - beta[j] * np.outer(k[j], k[j])) @ np.diag(np.exp(g[j]))
         for j in range(T)]
    o = np.zeros((T, dv))
    for t in range(T):
        acc = np.zeros(dv)
        for i in range(t + 1):
            Pm = np.eye(dk)
            for j in range(i + 1, t + 1):
                Pm = M[j] @ Pm
            acc += beta[i] * (q[t] @ Pm @ k[i]) * v[i]
        Pm = np.eye(dk)
        for j in range(t + 1):
            Pm = M[j] @ Pm
        o[t] = acc + q[t] @ Pm @ S0
    S = S0.copy()
    for t in range(T):
        S = M[t] @ S + beta[t] * np.outer(k[t], v[t])
    return o, S


def deltanet(q, k, v, beta, S0=None):
    """DeltaNet (page "Kimi K3论文：Kimi Linear", section 2): one online gradient
    step of size beta_t on 1/2 ||S^T k_t - v_t||^2, i.e.
    S_t = S_{t-1} - beta_t k_t (S_{t-1}^T k_t - v_t)^T, o_t = S_t^T q_t."""
    q, k, v, beta = (np.asarray(x, np.float64) for x in (q, k, v, beta))
    T, dk = q.shape
    dv = v.shape[1]
    S = np.zeros((dk, dv)) if S0 is None else np.array(S0, np.float64)
    o = np.zeros((T, dv))
    for t in range(T):
        grad = np.outer(k[t], S.T @ k[t] - v[t])
        S = S - beta[t] * grad
        o[t] = S.T @ q[t]
    return o, S


def gated_deltanet(q, k, v, log_a, beta, S0=None):
    """Gated DeltaNet (page "Kimi K3论文：Kimi Linear", section 2): a scalar gate
    per head and token, S_t = a_t (I - beta_t k_t k_t^T) S_{t-1} + beta_t k_t
    v_t^T.  ``log_a`` has shape [T]."""
    q, k, v, log_a, beta = (np.asarray(x, np.float64) for x in (q, k, v, log_a, beta))
    T, dk = q.shape
    dv = v.shape[1]
    S = np.zeros((dk, dv)) if S0 is None else np.array(S0, np.float64)
    o = np.zeros((T, dv))
    for t in range(T):
        S = np.exp(log_a[t]) * (S - beta[t] * np.outer(k[t], k[t] @ S)) \
            + beta[t] * np.outer(k[t], v[t])
        o[t] = S.T @ q[t]
    return o, S
