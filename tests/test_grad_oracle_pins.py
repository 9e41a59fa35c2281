"""Pins for the gradient oracle (no GPU).

``kda_ref.recurrent_grad`` (reverse mode through the fp64 recurrence of eq. (1)
on page "Kimi K3论文：Kimi Linear", section 3) is checked against things other
than itself: central finite differences of the forward oracle, torch autograd
through an independent torch transcription, closed forms for one token and for
beta = 0 (pure per-channel decay), linearity in the incoming gradients, the
chunk-boundary property that the backward pass of the chunked form relies on
(the gradient of a split sequence equals that of the whole when the second
half's dS0 is fed to the first half as dS_T), and padding tokens.  The mutation
tests at the end plant plausible mistakes in a Python copy of the reverse sweep
and check that the finite-difference pin catches each one.
"""
import numpy as np
import pytest

from oracle import kda_ref

NAMES = ("dq", "dk", "dv", "dg", "dbeta", "dS0")


def rand_case(rng, B, T, H, dk, dv, gscale=0.3, s0=True, beta_range=(0.0, 1.0)):
    q = rng.standard_normal((B, T, H, dk))
    k = rng.standard_normal((B, T, H, dk))
    q /= np.linalg.norm(q, axis=-1, keepdims=True)
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, T, H, dv))
    g = -gscale * np.log1p(np.exp(rng.standard_normal((B, T, H, dk))))
    beta = rng.uniform(*beta_range, size=(B, T, H))
    S0 = 0.5 * rng.standard_normal((B, H, dk, dv)) if s0 else None
    dO = rng.standard_normal((B, T, H, dv))
    dST = rng.standard_normal((B, H, dk, dv))
    return q, k, v, g, beta, S0, dO, dST


def relerr(x, ref):
    x, ref = np.asarray(x), np.asarray(ref)
    return float(np.max(np.abs(x - ref)) / max(np.max(np.abs(ref)), 1e-300))


def loss(q, k, v, g, beta, S0, dO, dST):
    o, S = kda_ref.recurrent(q, k, v, g, beta, S0)
    return float(np.sum(o * dO) + (0.0 if dST is None else np.sum(S * dST)))


def finite_difference(q, k, v, g, beta, S0, dO, dST, h=1e-6):
    """Central differences of the forward oracle's loss for every input entry."""
    args = [q, k, v, g, beta, S0]
    out = []
    for i, x in enumerate(args):
        d = np.zeros(x.shape)
        for idx in np.ndindex(*x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            ap, am = list(args), list(args)
            ap[i], am[i] = xp, xm
            d[idx] = (loss(*ap, dO, dST) - loss(*am, dO, dST)) / (2 * h)
        out.append(d)
    return out


def test_head_gate_gradient_is_the_channel_sum():
    """One decay per head and token (Gated DeltaNet): the gradient of that
    scalar, by central differences of the forward oracle with the decay copied
    to every channel, equals the per-channel gradient summed over channels."""
    rng = np.random.default_rng(21)
    q, k, v, _, beta, S0, dO, dST = rand_case(rng, 1, 4, 2, 3, 2)
    gh = -0.4 * np.log1p(np.exp(rng.standard_normal((1, 4, 2))))
    g = np.repeat(gh[..., None], 3, axis=-1)
    dg = kda_ref.recurrent_grad(q, k, v, g, beta, S0, dO, dST)[3]
    h = 1e-6
    fd = np.zeros(gh.shape)
    for idx in np.ndindex(*gh.shape):
        gp, gm = gh.copy(), gh.copy()
        gp[idx] += h
        gm[idx] -= h
        lp = loss(q, k, v, np.repeat(gp[..., None], 3, axis=-1), beta, S0, dO, dST)
        lm = loss(q, k, v, np.repeat(gm[..., None], 3, axis=-1), beta, S0, dO, dST)
        fd[idx] = (lp - lm) / (2 * h)
    assert relerr(dg.sum(axis=-1), fd) < 1e-7
    assert relerr(dg[..., 0], fd) > 1e-3      # a single channel is not enough

# ------------------------------------------------------- finite differences
@pytest.mark.parametrize("T", [1, 3, 9])
def test_matches_central_finite_differences(T):
    rng = np.random.default_rng(100 + T)
    q, k, v, g, beta, S0, dO, dST = rand_case(rng, 1, T, 2, 4, 3, gscale=0.6)
    grads = kda_ref.recurrent_grad(q, k, v, g, beta, S0, dO, dST)
    fd = finite_difference(q, k, v, g, beta, S0, dO, dST)
    for name, a, b in zip(NAMES, grads, fd):
        assert relerr(a, b) < 1e-7, name


def test_finite_differences_without_initial_state_or_final_gradient():
    rng = np.random.default_rng(7)
    q, k, v, g, beta, _, dO, _ = rand_case(rng, 2, 5, 1, 3, 4, gscale=0.4)
    grads = kda_ref.recurrent_grad(q, k, v, g, beta, None, dO, None)
    fd = finite_difference(q, k, v, g, beta, np.zeros((2, 1, 3, 4)), dO, None)
    for name, a, b in zip(NAMES, grads, fd):
        assert relerr(a, b) < 1e-7, name


# ----------------------------------------------------------------- autograd
def test_matches_torch_autograd_across_checkpoint_segments():
    """T = 150 crosses two checkpoint-segment boundaries of the C sweep."""
    rng = np.random.default_rng(3)
    q, k, v, g, beta, S0, dO, dST = rand_case(rng, 2, 150, 2, 16, 12, gscale=0.1)
    grads = kda_ref.recurrent_grad(q, k, v, g, beta, S0, dO, dST)
    for b in range(2):
        for h in range(2):
            ag = kda_ref.autograd_grad(q[b, :, h], k[b, :, h], v[b, :, h], g[b, :, h],
                                       beta[b, :, h], S0[b, h], dO[b, :, h], dST[b, h])
            mine = [x[b, :, h] for x in grads[:5]] + [grads[5][b, h]]
            for name, a, r in zip(NAMES, mine, ag):
                assert relerr(a, r) < 1e-12, (name, b, h)


# ------------------------------------------------------------- closed forms
def test_single_token_closed_form():
    """T = 1: S' = Diag(a) S0, o = S'^T q + beta (k.q) (v - S'^T k)."""
    rng = np.random.default_rng(11)
    q, k, v, g, beta, S0, dO, _ = rand_case(rng, 1, 1, 1, 5, 4)
    grads = kda_ref.recurrent_grad(q, k, v, g, beta, S0, dO, None)
    q1, k1, v1, g1, b1, do1, S = q[0, 0, 0], k[0, 0, 0], v[0, 0, 0], g[0, 0, 0], beta[0, 0, 0], dO[0, 0, 0], S0[0, 0]
    a = np.exp(g1)
    Sp = a[:, None] * S
    r = Sp.T @ k1
    kq = k1 @ q1
    w = v1 - r
    exp_dq = Sp @ do1 + b1 * (w @ do1) * k1
    exp_dk = b1 * (w @ do1) * q1 - b1 * kq * (Sp @ do1)
    exp_dv = b1 * kq * do1
    exp_dbeta = kq * (w @ do1)
    dSp = np.outer(q1 - b1 * kq * k1, do1)
    exp_dg = np.sum(dSp * Sp, axis=1)
    exp_dS0 = a[:, None] * dSp
    expected = (exp_dq, exp_dk, exp_dv, exp_dg, exp_dbeta, exp_dS0)
    got = [x[0, 0, 0] for x in grads[:5]] + [grads[5][0, 0]]
    for name, x, e in zip(NAMES, got, expected):
        assert relerr(x, e) < 1e-13, name


def test_beta_zero_closed_form():
    """beta = 0: S_t = Diag(e^{G_t}) S0 with G_t the running sum of g, so
    o_t[j] = sum_c q_t[c] e^{G_t[c]} S0[c, j]; k and v get no gradient and
    dg_s[c] = sum_{t >= s} q_t[c] e^{G_t[c]} (S0 dO_t)[c] + e^{G_T[c]} (S0 * dS_T)[c, :].sum()."""
    rng = np.random.default_rng(12)
    q, k, v, g, _, S0, dO, dST = rand_case(rng, 1, 7, 1, 4, 3, gscale=0.5)
    beta = np.zeros((1, 7, 1))
    dq, dk, dv, dg, dbeta, dS0 = kda_ref.recurrent_grad(q, k, v, g, beta, S0, dO, dST)
    assert np.all(dk == 0) and np.all(dv == 0)
    G = np.cumsum(g[0, :, 0], axis=0)
    S = S0[0, 0]
    per_t = q[0, :, 0] * np.exp(G) * (dO[0, :, 0] @ S.T)            # [t, c]
    final = np.exp(G[-1]) * np.sum(S * dST[0, 0], axis=1)           # [c]
    exp_dg = np.cumsum(per_t[::-1], axis=0)[::-1] + final[None, :]
    assert relerr(dg[0, :, 0], exp_dg) < 1e-13
    exp_dq = np.exp(G) * (dO[0, :, 0] @ S.T)
    assert relerr(dq[0, :, 0], exp_dq) < 1e-13
    exp_dS0 = (q[0, :, 0] * np.exp(G)).T @ dO[0, :, 0] + np.exp(G[-1])[:, None] * dST[0, 0]
    assert relerr(dS0[0, 0], exp_dS0) < 1e-13


# --------------------------------------------------------------- structure
def test_linear_in_incoming_gradients():
    rng = np.random.default_rng(13)
    q, k, v, g, beta, S0, dO, dST = rand_case(rng, 1, 20, 2, 6, 5)
    dO2, dST2 = rng.standard_normal(dO.shape), rng.standard_normal(dST.shape)
    g1 = kda_ref.recurrent_grad(q, k, v, g, beta, S0, dO, dST)
    g2 = kda_ref.recurrent_grad(q, k, v, g, beta, S0, dO2, dST2)
    g3 = kda_ref.recurrent_grad(q, k, v, g, beta, S0, 2 * dO - 3 * dO2, 2 * dST - 3 * dST2)
    for a, b, c in zip(g1, g2, g3):
        assert relerr(c, 2 * a - 3 * b) < 1e-12


@pytest.mark.parametrize("split", [1, 64, 77])
def test_split_sequence_carries_the_state_gradient(split):
    """Run the second part with the state the first part ends in; its dS0 fed
    as dS_T of the first part gives the whole sequence's gradients."""
    rng = np.random.default_rng(14)
    q, k, v, g, beta, S0, dO, dST = rand_case(rng, 1, 130, 1, 8, 8, gscale=0.1)
    full = kda_ref.recurrent_grad(q, k, v, g, beta, S0, dO, dST)
    a, b = slice(0, split), slice(split, None)
    _, S_mid = kda_ref.recurrent(q[:, a], k[:, a], v[:, a], g[:, a], beta[:, a], S0)
    second = kda_ref.recurrent_grad(q[:, b], k[:, b], v[:, b], g[:, b], beta[:, b], S_mid, dO[:, b], dST)
    first = kda_ref.recurrent_grad(q[:, a], k[:, a], v[:, a], g[:, a], beta[:, a], S0, dO[:, a], second[5])
    for i in range(5):
        joined = np.concatenate([first[i], second[i]], axis=1)
        assert relerr(joined, full[i]) < 1e-12, NAMES[i]
    assert relerr(first[5], full[5]) < 1e-12


def test_padding_tokens_change_nothing():
    """Tokens with k = v = 0, beta = 0, g = 0 and no incoming gradient leave the
    state alone, so the real tokens' gradients are unchanged; the padded tokens'
    dq, dk, dv and dbeta are zero, and their dg is the row-wise product of the
    final state and its incoming gradient (the gate still scales the state)."""
    rng = np.random.default_rng(15)
    q, k, v, g, beta, S0, dO, dST = rand_case(rng, 1, 10, 1, 5, 4)
    base = kda_ref.recurrent_grad(q, k, v, g, beta, S0, dO, dST)
    pad = lambda x, val=0.0: np.concatenate([x, np.full((1, 6) + x.shape[2:], val)], axis=1)
    qp = pad(q, 0.3)
    padded = kda_ref.recurrent_grad(qp, pad(k), pad(v), pad(g), pad(beta), S0, pad(dO), dST)
    for i in range(5):
        assert relerr(padded[i][:, :10], base[i]) < 1e-13, NAMES[i]
        if i != 3:
            assert np.all(padded[i][:, 10:] == 0), NAMES[i]
    _, S_T = kda_ref.recurrent(q, k, v, g, beta, S0)
    row = np.sum(S_T[0, 0] * dST[0, 0], axis=1)
    assert relerr(padded[3][0, 10:, 0], np.broadcast_to(row, (6, 5))) < 1e-13
    assert relerr(padded[5], base[5]) < 1e-13


def test_heads_independent_and_thread_count_deterministic():
    rng = np.random.default_rng(16)
    q, k, v, g, beta, S0, dO, dST = rand_case(rng, 2, 30, 3, 6, 5)
    one = kda_ref.recurrent_grad(q, k, v, g, beta, S0, dO, dST, nthreads=1)
    many = kda_ref.recurrent_grad(q, k, v, g, beta, S0, dO, dST, nthreads=4)
    for a, b in zip(one, many):
        assert np.array_equal(a, b)
    sl = lambda x: x[1:2, :, 2:3]
    alone = kda_ref.recurrent_grad(sl(q), sl(k), sl(v), sl(g), sl(beta), S0[1:2, 2:3], sl(dO), dST[1:2, 2:3])
    for i in range(5):
        assert np.array_equal(alone[i], sl(one[i]))
    assert np.array_equal(alone[5], one[5][1:2, 2:3])


# ---------------------------------------------------------------- mutations
def _grad_mutant(kind):
    """A Python copy of the reverse sweep with one plausible mistake planted."""
    def run(q, k, v, g, beta, S0, dO, dST):
        T, dk = q.shape
        dv = v.shape[1]
        states = [S0.copy()]
        for t in range(T):
            Sp = np.exp(g[t])[:, None] * states[-1]
            u = beta[t] * (v[t] - Sp.T @ k[t])
            states.append(Sp + np.outer(k[t], u))
        D = dST.copy()
        dq, dk_, dg = np.zeros((T, dk)), np.zeros((T, dk)), np.zeros((T, dk))
        dv_, dbeta = np.zeros((T, dv)), np.zeros(T)
        for t in range(T - 1, -1, -1):
            a = np.exp(g[t])
            Sp = a[:, None] * states[t]
            r = Sp.T @ k[t]
            u = beta[t] * (v[t] - r)
            St = states[t + 1]
            dq[t] = (Sp if kind == "read_before_write" else St) @ dO[t]
            D = D + np.outer(q[t], dO[t])
            du = D.T @ k[t]
            dk_[t] = D @ u
            dbeta[t] = du @ ((v[t] if kind == "dbeta_drops_r" else v[t] - r))
            dv_[t] = beta[t] * du
            dr = (1 if kind == "dr_sign" else -1) * beta[t] * du
            if kind != "no_key_through_r":
                dk_[t] += Sp @ dr
            D = D + np.outer(k[t], dr)
            dg[t] = np.sum(D * (states[t] if kind == "dg_uses_old_state" else Sp), axis=1)
            if kind != "no_decay_on_carry":
                D = a[:, None] * D
        return dq, dk_, dv_, dg, dbeta, D
    return run


@pytest.mark.parametrize("kind", ["read_before_write", "dbeta_drops_r", "dr_sign",
                                  "no_key_through_r", "dg_uses_old_state", "no_decay_on_carry"])
def test_pins_catch_planted_mistakes(kind):
    rng = np.random.default_rng(17)
    q, k, v, g, beta, S0, dO, dST = rand_case(rng, 1, 4, 1, 3, 3, gscale=0.6)
    args = [x[0, :, 0] for x in (q, k, v, g)] + [beta[0, :, 0], S0[0, 0], dO[0, :, 0], dST[0, 0]]
    mutant = _grad_mutant(kind)(*args)
    fd = finite_difference(q, k, v, g, beta, S0, dO, dST)
    fd = [x[0, :, 0] for x in fd[:5]] + [fd[5][0, 0]]
    assert max(relerr(m, f) for m, f in zip(mutant, fd)) > 1e-4
    clean = _grad_mutant("none")(*args)
    assert max(relerr(c, f) for c, f in zip(clean, fd)) < 1e-7
