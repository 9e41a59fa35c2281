"""Pins for the CPU oracle (no GPU).

The oracle (oracle/kda_ref.c, the sequential fp64 recurrence of eq. (1) on page
"Kimi K3论文：Kimi Linear", section 3) is checked against things other than
itself: a hand-worked example, closed forms, the reductions to DeltaNet and
Gated DeltaNet, the delta-rule retrieval identity, and independent cross-forms
taken from other passages (DPLR rewrite, chunked Proposition, product form).
The mutation tests at the end plant plausible mistakes in a copy of the
recurrence and check that these pins catch each one.
"""
import json
import os

import numpy as np
import pytest

from oracle import kda_ref

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rand_inputs(rng, B, T, H, dk, dv, gscale=0.1, s0=True, beta_range=(0.0, 1.0)):
    q = rng.standard_normal((B, T, H, dk))
    k = rng.standard_normal((B, T, H, dk))
    q /= np.linalg.norm(q, axis=-1, keepdims=True)
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, T, H, dv))
    g = -gscale * np.log1p(np.exp(rng.standard_normal((B, T, H, dk))))
    beta = rng.uniform(*beta_range, size=(B, T, H))
    S0 = 0.3 * rng.standard_normal((B, H, dk, dv)) if s0 else None
    return q, k, v, g, beta, S0


def relerr(x, ref):
    x, ref = np.asarray(x), np.asarray(ref)
    return float(np.max(np.abs(x - ref)) / max(np.max(np.abs(ref)), 1e-300))


# --------------------------------------------------------------------- golden
def test_hand_worked_example():
    """tests/golden/kda_hand_example.json: eq. (1) worked by hand (d = 2, T = 3)."""
    with open(os.path.join(GOLDEN, "kda_hand_example.json")) as f:
        ex = json.load(f)
    sh = lambda a: np.asarray(a, np.float64)[None, :, None]  # [1, T, 1, d]
    q, k, v = sh(ex["q"]), sh(ex["k"]), sh(ex["v"])
    g = np.log(sh(ex["alpha"]))
    beta = np.asarray(ex["beta"], np.float64)[None, :, None]
    o, S = kda_ref.recurrent(q, k, v, g, beta)
    np.testing.assert_allclose(o[0, :, 0], ex["o"], atol=1e-14)
    np.testing.assert_allclose(S[0, 0], ex["S_T"], atol=1e-14)
    for form in (kda_ref.dplr_form, kda_ref.chunked_form, kda_ref.product_form):
        o2, S2 = kda_ref.per_head(form, q, k, v, g, beta)
        np.testing.assert_allclose(o2[0, :, 0], ex["o"], atol=1e-14)
        np.testing.assert_allclose(S2[0, 0], ex["S_T"], atol=1e-14)


# ------------------------------------------------------------ closed forms
def test_beta_zero_is_pure_per_channel_decay():
    """beta = 0: S_T = Diag(exp(sum_t g_t)) S0 and o_t = S0^T (exp(G_t) * q_t)."""
    rng = np.random.default_rng(1)
    q, k, v, g, beta, S0 = rand_inputs(rng, 2, 37, 3, 16, 12)
    beta[:] = 0.0
    o, S = kda_ref.recurrent(q, k, v, g, beta, S0)
    G = np.cumsum(g, axis=1)                                    # [B,T,H,dk]
    S_ref = np.exp(G[:, -1])[..., None] * S0
    o_ref = np.einsum("bhcj,bthc->bthj", S0, np.exp(G) * q)
    assert relerr(S, S_ref) < 1e-13
    assert relerr(o, o_ref) < 1e-13


def test_zero_initial_state_and_zero_values_give_zero():
    rng = np.random.default_rng(2)
    q, k, v, g, beta, _ = rand_inputs(rng, 1, 20, 2, 8, 8, s0=False)
    o, S = kda_ref.recurrent(q, k, np.zeros_like(v), g, beta, None)
    assert np.all(o == 0.0) and np.all(S == 0.0)


def test_basis_keys_decouple_rows():
    """k_t = e_{c_t}: row c of S evolves as S[c] <- alpha_c S[c], and when
    c = c_t additionally S[c] <- (1 - beta) S[c] + beta v_t (scalar closed form)."""
    rng = np.random.default_rng(3)
    T, dk, dv = 50, 6, 5
    c_t = rng.integers(0, dk, size=T)
    k = np.zeros((1, T, 1, dk))
    k[0, np.arange(T), 0, c_t] = 1.0
    q = rng.standard_normal((1, T, 1, dk))
    v = rng.standard_normal((1, T, 1, dv))
    g = -0.2 * rng.uniform(size=(1, T, 1, dk))
    beta = rng.uniform(size=(1, T, 1))
    S0 = rng.standard_normal((1, 1, dk, dv))
    o, S = kda_ref.recurrent(q, k, v, g, beta, S0)
    rows = S0[0, 0].copy()
    for t in range(T):
        rows = np.exp(g[0, t, 0])[:, None] * rows
        c, b = c_t[t], beta[0, t, 0]
        rows[c] = (1 - b) * rows[c] + b * v[0, t, 0]
        np.testing.assert_allclose(o[0, t, 0], rows.T @ q[0, t, 0], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(S[0, 0], rows, rtol=1e-12, atol=1e-13)


def test_retrieval_identity():
    """With ||k_t|| = 1 the write makes S_t^T k_t = (1 - beta_t) S'^T k_t + beta_t v_t
    (S' = Diag(alpha_t) S_{t-1}); with beta_t = 1 the value is stored exactly."""
    rng = np.random.default_rng(4)
    q, k, v, g, beta, S0 = rand_inputs(rng, 1, 12, 1, 16, 9)
    beta[0, 7, 0] = 1.0
    for t in range(1, 12):
        _, S_prev = kda_ref.recurrent(q[:, :t], k[:, :t], v[:, :t], g[:, :t], beta[:, :t], S0)
        _, S_t = kda_ref.recurrent(q[:, :t + 1], k[:, :t + 1], v[:, :t + 1], g[:, :t + 1],
                                   beta[:, :t + 1], S0)
        kt, b = k[0, t, 0], beta[0, t, 0]
        Sp = np.exp(g[0, t, 0])[:, None] * S_prev[0, 0]
        lhs = S_t[0, 0].T @ kt
        rhs = (1 - b) * (Sp.T @ kt) + b * v[0, t, 0]
        np.testing.assert_allclose(lhs, rhs, rtol=1e-12, atol=1e-12)
        if t == 7:
            np.testing.assert_allclose(lhs, v[0, t, 0], rtol=1e-12, atol=1e-12)


# -------------------------------------------------------------- reductions
def test_alpha_one_reduces_to_deltanet():
    rng = np.random.default_rng(5)
    q, k, v, g, beta, S0 = rand_inputs(rng, 1, 40, 2, 16, 12)
    g[:] = 0.0
    o, S = kda_ref.recurrent(q, k, v, g, beta, S0)
    for h in range(2):
        o2, S2 = kda_ref.deltanet(q[0, :, h], k[0, :, h], v[0, :, h], beta[0, :, h], S0[0, h])
        assert relerr(o[0, :, h], o2) < 1e-13 and relerr(S[0, h], S2) < 1e-13


def test_scalar_alpha_reduces_to_gated_deltanet():
    rng = np.random.default_rng(6)
    q, k, v, _, beta, S0 = rand_inputs(rng, 1, 40, 2, 16, 12)
    log_a = -0.3 * rng.uniform(size=(1, 40, 2))
    g = np.repeat(log_a[..., None], 16, axis=-1)
    o, S = kda_ref.recurrent(q, k, v, g, beta, S0)
    for h in range(2):
        o2, S2 = kda_ref.gated_deltanet(q[0, :, h], k[0, :, h], v[0, :, h], log_a[0, :, h],
                                        beta[0, :, h], S0[0, h])
        assert relerr(o[0, :, h], o2) < 1e-13 and relerr(S[0, h], S2) < 1e-13


# ------------------------------------------------------------- cross-forms
@pytest.mark.parametrize("T", [1, 7, 63, 64, 65, 200])
def test_dplr_and_chunked_forms_equal_recurrence(T):
    rng = np.random.default_rng(100 + T)
    q, k, v, g, beta, S0 = rand_inputs(rng, 1, T, 2, 16, 12, gscale=0.5)
    o, S = kda_ref.recurrent(q, k, v, g, beta, S0)
    o2, S2 = kda_ref.per_head(kda_ref.dplr_form, q, k, v, g, beta, S0)
    assert relerr(o2, o) < 1e-12 and relerr(S2, S) < 1e-12
    for C in sorted({1, 7, 64, T}):
        o3, S3 = kda_ref.per_head(kda_ref.chunked_form, q, k, v, g, beta, S0, C=C)
        assert relerr(o3, o) < 1e-11, C
        assert relerr(S3, S) < 1e-11, C


def test_full_head_dim_forms_agree():
    """d_k = d_v = 128, C = 64, ragged tail: the chunked form equals the oracle."""
    rng = np.random.default_rng(7)
    q, k, v, g, beta, S0 = rand_inputs(rng, 1, 150, 1, 128, 128, gscale=0.1)
    o, S = kda_ref.recurrent(q, k, v, g, beta, S0)
    o3, S3 = kda_ref.per_head(kda_ref.chunked_form, q, k, v, g, beta, S0, C=64)
    assert relerr(o3, o) < 1e-11 and relerr(S3, S) < 1e-11


def test_proposition_states_match_recurrence():
    rng = np.random.default_rng(8)
    L = 16
    q, k, v, g, beta, S0 = rand_inputs(rng, 1, L, 1, 8, 6, gscale=0.5)
    o_p, states = kda_ref.proposition_states(q[0, :, 0], k[0, :, 0], v[0, :, 0],
                                             g[0, :, 0], beta[0, :, 0], S0[0, 0])
    o, _ = kda_ref.recurrent(q, k, v, g, beta, S0)
    assert relerr(o_p, o[0, :, 0]) < 1e-12
    for r in (0, 5, L - 1):
        _, S_r = kda_ref.recurrent(q[:, :r + 1], k[:, :r + 1], v[:, :r + 1], g[:, :r + 1],
                                   beta[:, :r + 1], S0)
        assert relerr(states[r], S_r[0, 0]) < 1e-12


@pytest.mark.parametrize("T", [1, 5, 11])
def test_product_form_equals_recurrence(T):
    rng = np.random.default_rng(200 + T)
    q, k, v, g, beta, S0 = rand_inputs(rng, 1, T, 1, 6, 5, gscale=0.7)
    o, S = kda_ref.recurrent(q, k, v, g, beta, S0)
    o2, S2 = kda_ref.per_head(kda_ref.product_form, q, k, v, g, beta, S0)
    assert relerr(o2, o) < 1e-12 and relerr(S2, S) < 1e-12


def test_forward_substitution_closed_form():
    """I + A with A = -c on the first subdiagonal has inverse c^(i-j) (i >= j)."""
    C, c = 64, 0.9
    A = np.zeros((C, C))
    A[np.arange(1, C), np.arange(C - 1)] = -c
    Tm = kda_ref.forward_substitution(A)
    i, j = np.indices((C, C))
    ref = np.where(i >= j, c ** (i - j).astype(float), 0.0)
    np.testing.assert_allclose(Tm, ref, rtol=1e-13, atol=1e-15)
    rng = np.random.default_rng(9)
    A = np.tril(rng.standard_normal((C, C)) * 0.1, -1)
    Tm = kda_ref.forward_substitution(A)
    np.testing.assert_allclose(Tm @ (np.eye(C) + A), np.eye(C), atol=1e-12)


def test_mask_with_diagonal_breaks_the_chunked_form():
    """The page prints one mask (diagonal kept).  Using it for Akk instead of the
    strict lower triangle gives O(1) errors, so the strict reading is forced."""
    rng = np.random.default_rng(10)
    q, k, v, g, beta, S0 = rand_inputs(rng, 1, 64, 1, 16, 8)
    q1, k1, v1, g1, b1 = q[0, :, 0], k[0, :, 0], v[0, :, 0], g[0, :, 0], beta[0, :, 0]
    G = np.cumsum(g1, 0)
    D = np.exp(G[:, None, :] - G[None, :, :])
    kk = np.einsum("rc,ic,ric->ri", k1, k1, D)
    A_wrong = b1[:, None] * np.tril(kk, 0)           # diagonal kept
    T_wrong = np.linalg.inv(np.eye(64) + A_wrong)
    T_right = kda_ref.forward_substitution(b1[:, None] * np.tril(kk, -1))
    W_r = T_right @ (b1[:, None] * np.exp(G) * k1)
    W_w = T_wrong @ (b1[:, None] * np.exp(G) * k1)
    assert relerr(W_w, W_r) > 0.1


# --------------------------------------------------------------- properties
def test_linearity_in_values_and_initial_state():
    rng = np.random.default_rng(11)
    q, k, v1, g, beta, S01 = rand_inputs(rng, 1, 30, 2, 16, 8)
    v2 = rng.standard_normal(v1.shape)
    S02 = rng.standard_normal(S01.shape)
    a, b = 0.7, -1.3
    o1, S1 = kda_ref.recurrent(q, k, v1, g, beta, S01)
    o2, S2 = kda_ref.recurrent(q, k, v2, g, beta, S02)
    o3, S3 = kda_ref.recurrent(q, k, a * v1 + b * v2, g, beta, a * S01 + b * S02)
    assert relerr(o3, a * o1 + b * o2) < 1e-12 and relerr(S3, a * S1 + b * S2) < 1e-12


def test_split_and_resume():
    rng = np.random.default_rng(12)
    q, k, v, g, beta, S0 = rand_inputs(rng, 2, 90, 2, 16, 8)
    o, S = kda_ref.recurrent(q, k, v, g, beta, S0)
    t1 = 37
    oa, Sa = kda_ref.recurrent(q[:, :t1], k[:, :t1], v[:, :t1], g[:, :t1], beta[:, :t1], S0)
    ob, Sb = kda_ref.recurrent(q[:, t1:], k[:, t1:], v[:, t1:], g[:, t1:], beta[:, t1:], Sa)
    assert relerr(np.concatenate([oa, ob], axis=1), o) < 1e-13 and relerr(Sb, S) < 1e-13


def test_segment_summaries_compose():
    """The state after a run of tokens is an affine map of the state before it
    (the Proposition S_r = P_r S_0 + H_r of page "Kimi Linear：高效注意力机制
    在长序列处理中的创新应用", section 2.1, taken over a whole segment): its
    offset E is the end state from zero, and its matrix P is the end state of
    the identity run with zero values.  Composing S_{j+1} = P_j S_j + E_j over
    segments, then running every segment from its entry state, reproduces the
    one-pass outputs and final state (the segmented state scan's plan)."""
    rng = np.random.default_rng(16)
    B, T, H, dk, dv = 1, 70, 2, 16, 8
    q, k, v, g, beta, S0 = rand_inputs(rng, B, T, H, dk, dv)
    o, S = kda_ref.recurrent(q, k, v, g, beta, S0)
    cuts = [0, 17, 40, 52, T]
    Sj, outs = S0, []
    eye = np.broadcast_to(np.eye(dk), (B, H, dk, dk)).copy()
    for a, b in zip(cuts[:-1], cuts[1:]):
        sl = lambda x: x[:, a:b]
        oj, _ = kda_ref.recurrent(sl(q), sl(k), sl(v), sl(g), sl(beta), Sj)
        outs.append(oj)
        _, E = kda_ref.recurrent(sl(q), sl(k), sl(v), sl(g), sl(beta), None)
        zero_v = np.zeros((B, b - a, H, dk))
        _, P = kda_ref.recurrent(sl(q), sl(k), zero_v, sl(g), sl(beta), eye)
        Sj = P @ Sj + E
    assert relerr(np.concatenate(outs, axis=1), o) < 1e-12 and relerr(Sj, S) < 1e-12


def test_padding_tokens_are_identity():
    rng = np.random.default_rng(13)
    q, k, v, g, beta, S0 = rand_inputs(rng, 1, 20, 1, 16, 8)
    pad = lambda a, n=5: np.concatenate([a, np.zeros((1, n) + a.shape[2:])], axis=1)
    _, S = kda_ref.recurrent(q, k, v, g, beta, S0)
    o2, S2 = kda_ref.recurrent(pad(q), pad(k), pad(v), pad(g), pad(beta), S0)
    assert np.array_equal(S2, S) and np.all(o2[:, 20:] == 0.0)


def test_value_columns_are_separable():
    rng = np.random.default_rng(14)
    q, k, v, g, beta, S0 = rand_inputs(rng, 1, 40, 2, 16, 16)
    o, S = kda_ref.recurrent(q, k, v, g, beta, S0)
    cols = slice(4, 12)
    o2, S2 = kda_ref.recurrent(q, k, v[..., cols], g, beta, S0[..., cols])
    assert relerr(o2, o[..., cols]) < 1e-13 and relerr(S2, S[..., cols]) < 1e-13


def test_heads_and_batches_are_independent_and_threads_deterministic():
    rng = np.random.default_rng(15)
    q, k, v, g, beta, S0 = rand_inputs(rng, 3, 25, 4, 8, 8)
    o, S = kda_ref.recurrent(q, k, v, g, beta, S0, nthreads=1)
    o4, S4 = kda_ref.recurrent(q, k, v, g, beta, S0, nthreads=4)
    assert np.array_equal(o, o4) and np.array_equal(S, S4)
    o1, S1 = kda_ref.recurrent(q[1:2, :, 2:3], k[1:2, :, 2:3], v[1:2, :, 2:3],
                               g[1:2, :, 2:3], beta[1:2, :, 2:3], S0[1:2, 2:3])
    assert np.array_equal(o1[0, :, 0], o[1, :, 2]) and np.array_equal(S1[0, 0], S[1, 2])


# ------------------------------------------------------------------ mutations
def _mutant(kind):
    """A copy of the recurrence with one plausible mistake planted in it."""
    def run(q, k, v, g, beta, S0):
        T, dk = q.shape
        S = S0.copy()
        o = np.zeros((T, v.shape[1]))
        for t in range(T):
            a = np.exp(g[t])
            if kind == "gate_after_householder":
                S = a[:, None] * (S - beta[t] * np.outer(k[t], k[t] @ S)) + beta[t] * np.outer(k[t], v[t])
            else:
                Sp = a[:, None] * S
                if kind == "gate_on_columns":
                    Sp = S * np.resize(a, S.shape[1])[None, :]
                r = Sp.T @ k[t]
                if kind == "sign_flip":
                    r = -r
                u = beta[t] * (v[t] - r)
                if kind == "no_beta":
                    u = v[t] - r
                S = Sp + np.outer(k[t], u)
            o[t] = S.T @ (k[t] if kind == "read_with_key" else q[t])
        return o, S
    return run


@pytest.mark.parametrize("kind", ["gate_after_householder", "gate_on_columns", "sign_flip",
                                  "no_beta", "read_with_key"])
def test_pins_catch_planted_mistakes(kind):
    """Each planted mistake must break at least one pin that the oracle passes."""
    rng = np.random.default_rng(16)
    q, k, v, g, beta, S0 = rand_inputs(rng, 1, 20, 1, 8, 6, gscale=0.8)
    args = (q[0, :, 0], k[0, :, 0], v[0, :, 0], g[0, :, 0], beta[0, :, 0], S0[0, 0])
    o_m, S_m = _mutant(kind)(*args)
    o_d, S_d = kda_ref.dplr_form(*args)
    o_c, S_c = kda_ref.chunked_form(*args, C=7)
    caught_dplr = relerr(o_m, o_d) > 1e-6 or relerr(S_m, S_d) > 1e-6
    caught_chunk = relerr(o_m, o_c) > 1e-6 or relerr(S_m, S_c) > 1e-6
    assert caught_dplr and caught_chunk
    o, S = kda_ref.recurrent(q, k, v, g, beta, S0)
    assert relerr(o[0, :, 0], o_d) < 1e-12 and relerr(S[0, 0], S_d) < 1e-12
