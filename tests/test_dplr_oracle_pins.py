"""Pins for the DPLR oracle (no GPU).

``dplr_ref.recurrent`` (the diagonal-plus-low-rank recurrence of page "Kimi
K3论文：Kimi Linear", section 4) is checked against: the KDA oracle under the
page's own mapping a = beta k, b = alpha * k; the closed form of gated linear
attention when a = 0; the product of the explicit d_k x d_k transition
matrices.  ``dplr_ref.chunked_head`` (the chunkwise form the GPU kernels
follow) is checked against the recurrence at several chunk sizes and ragged
lengths, and the mutation test plants plausible mistakes in a copy of it and
checks that the recurrence pin catches each one.
"""
import numpy as np
import pytest

from oracle import dplr_ref, kda_ref


def rand_dplr(rng, T, dk=6, dv=5, gscale=0.3, s0=True):
    nrm = lambda x: x / np.linalg.norm(x, axis=-1, keepdims=True)
    q, k, ka, kb = (nrm(rng.standard_normal((T, dk))) for _ in range(4))
    v = rng.standard_normal((T, dv))
    g = -gscale * np.log1p(np.exp(rng.standard_normal((T, dk))))
    beta = rng.uniform(0, 1, size=T)
    a = beta[:, None] * ka
    b = np.exp(g) * kb
    S0 = 0.5 * rng.standard_normal((dk, dv)) if s0 else None
    return q, k, v, a, b, g, S0


def relerr(x, ref):
    return float(np.max(np.abs(np.asarray(x) - ref)) / max(np.max(np.abs(ref)), 1e-300))


def test_reduces_to_kda_under_the_pages_mapping():
    """a = beta k, b = alpha * k and the write beta k v^T give eq. (1)."""
    rng = np.random.default_rng(0)
    B, T, H, dk, dv = 1, 40, 2, 8, 6
    q = rng.standard_normal((B, T, H, dk))
    k = rng.standard_normal((B, T, H, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, T, H, dv))
    g = -0.2 * np.log1p(np.exp(rng.standard_normal((B, T, H, dk))))
    beta = rng.uniform(0, 1, size=(B, T, H))
    S0 = rng.standard_normal((B, H, dk, dv))
    o_ref, S_ref = kda_ref.recurrent(q, k, v, g, beta, S0)
    bk = beta[..., None] * k
    o, S = dplr_ref.recurrent(q, bk, v, bk, np.exp(g) * k, g, S0)
    assert relerr(o, o_ref) < 1e-12 and relerr(S, S_ref) < 1e-12


def test_no_low_rank_term_is_gated_linear_attention():
    """a = 0: o_t = sum_{i<=t} (q_t * e^{G_t - G_i}) . k_i v_i + (e^{G_t} q_t)^T S0."""
    rng = np.random.default_rng(1)
    q, k, v, a, b, g, S0 = rand_dplr(rng, 23)
    o, _ = dplr_ref.recurrent_head(q, k, v, np.zeros_like(a), b, g, S0)
    G = np.cumsum(g, axis=0)
    ref = np.zeros_like(o)
    for t in range(23):
        ref[t] = (np.exp(G[t]) * q[t]) @ S0
        for i in range(t + 1):
            ref[t] += np.dot(q[t] * np.exp(G[t] - G[i]), k[i]) * v[i]
    assert relerr(o, ref) < 1e-12


def test_product_of_transition_matrices():
    """S_T = M_T ... M_1 S0 + sum_i M_T ... M_{i+1} k_i v_i^T with the dense
    transitions M_t = Diag(alpha_t) - a_t b_t^T, and o_t = S_t^T q_t."""
    rng = np.random.default_rng(2)
    T = 17
    q, k, v, a, b, g, S0 = rand_dplr(rng, T)
    o, S = dplr_ref.recurrent_head(q, k, v, a, b, g, S0)
    M = [np.diag(np.exp(g[t])) - np.outer(a[t], b[t]) for t in range(T)]

    def prod(lo, hi):                 # M_hi ... M_{lo+1} (0-based: M[lo] .. M[hi-1])
        P = np.eye(q.shape[1])
        for t in range(lo, hi):
            P = M[t] @ P
        return P

    for t in (0, 5, T - 1):
        St = prod(0, t + 1) @ S0 + sum(prod(i + 1, t + 1) @ np.outer(k[i], v[i]) for i in range(t + 1))
        assert relerr(o[t], St.T @ q[t]) < 1e-12
    assert relerr(S, prod(0, T) @ S0 + sum(prod(i + 1, T) @ np.outer(k[i], v[i]) for i in range(T))) < 1e-12


@pytest.mark.parametrize("T,C", [(1, 64), (5, 64), (64, 64), (65, 64), (130, 64), (50, 16), (23, 7)])
def test_chunked_form_equals_the_recurrence(T, C):
    rng = np.random.default_rng(10 + T + C)
    q, k, v, a, b, g, S0 = rand_dplr(rng, T, dk=8, dv=6)
    o, S = dplr_ref.recurrent_head(q, k, v, a, b, g, S0)
    oc, Sc = dplr_ref.chunked_head(q, k, v, a, b, g, S0, C=C)
    assert relerr(oc, o) < 1e-12 and relerr(Sc, S) < 1e-12


def test_linear_in_values_and_initial_state():
    rng = np.random.default_rng(3)
    q, k, v1, a, b, g, S1 = rand_dplr(rng, 30)
    _, _, v2, _, _, _, S2 = rand_dplr(rng, 30)
    o1, s1 = dplr_ref.recurrent_head(q, k, v1, a, b, g, S1)
    o2, s2 = dplr_ref.recurrent_head(q, k, v2, a, b, g, S2)
    o3, s3 = dplr_ref.recurrent_head(q, k, 2 * v1 - v2, a, b, g, 2 * S1 - S2)
    assert relerr(o3, 2 * o1 - o2) < 1e-12 and relerr(s3, 2 * s1 - s2) < 1e-12


def _chunked_variant(q, k, v, a, b, g, S0, mistake, C=8):
    """The chunked form with one planted mistake (test-only copy)."""
    T, dk = q.shape
    S = S0.copy()
    o = np.zeros((T, v.shape[1]))
    for s in range(0, T, C):
        e = min(s + C, T)
        Q, K, V, A, Bv, Gs = q[s:e], k[s:e], v[s:e], a[s:e], b[s:e], g[s:e]
        G = np.cumsum(Gs, axis=0)
        Gprev = G if mistake == "inclusive_read_decay" else G - Gs
        Dqk = np.exp(G[:, None, :] - G[None, :, :])
        Dbk = np.exp(Gprev[:, None, :] - G[None, :, :])
        A_qk = np.tril(np.einsum("rc,ic,ric->ri", Q, K, Dqk), 0)
        A_qa = np.tril(np.einsum("rc,ic,ric->ri", Q, A, Dqk), -1 if mistake == "strict_qa" else 0)
        A_bk = np.tril(np.einsum("rc,ic,ric->ri", Bv, K, Dbk), -1)
        A_ba = np.tril(np.einsum("rc,ic,ric->ri", Bv, A, Dbk), -1)
        if mistake == "swapped_ba":                     # a and b exchanged
            A_ba = np.tril(np.einsum("rc,ic,ric->ri", A, Bv, Dbk), -1)
        Tm = kda_ref.forward_substitution(A_ba)
        U = Tm @ ((np.exp(Gprev) * Bv) @ S + A_bk @ V)
        sign = 1.0 if mistake == "sign_qa" else -1.0
        o[s:e] = (np.exp(G) * Q) @ S + (0 if mistake == "no_intra_kv" else A_qk @ V) + sign * A_qa @ U
        Kt = np.exp(G[-1][None, :] - G)
        S = np.exp(G[-1])[:, None] * S + (Kt * K).T @ V - (Kt * A).T @ U
    return o, S


@pytest.mark.parametrize("mistake", ["inclusive_read_decay", "strict_qa", "swapped_ba", "sign_qa",
                                     "no_intra_kv"])
def test_planted_mistakes_are_caught(mistake):
    rng = np.random.default_rng(4)
    q, k, v, a, b, g, S0 = rand_dplr(rng, 20, gscale=0.8)
    o, S = dplr_ref.recurrent_head(q, k, v, a, b, g, S0)
    assert relerr(_chunked_variant(q, k, v, a, b, g, S0, None)[0], o) < 1e-12
    assert relerr(_chunked_variant(q, k, v, a, b, g, S0, mistake)[0], o) > 1e-4
