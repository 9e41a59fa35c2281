"""Pins for the layer oracle (oracle/kda_layer_ref.py), no GPU.

The layer of page "Kimi K3论文：Kimi Linear", section 3 (projections, causal
ShortConv, Swish, L2Norm, the decay and write gates, head RMSNorm and the
sigmoid output gate around eq. (1)) is checked against library routines
(numpy's convolution, scipy's logistic function), closed forms
(exp(-softplus(u)) = sigmoid(-u); one token from a zero state gives
o = beta (k.q) v), structural facts (causality, independent sequences,
orientation of [out, in] weights via permutation matrices) and the
invariants of the norms.  The mutation test at the end plants plausible
mistakes in a copy of the oracle's source and checks that some pin fails.
"""
import sys
import types

import numpy as np
import pytest
from scipy.special import expit

from oracle import kda_layer_ref

H, D, DM, RANK = 2, 4, 8, 3          # heads, head dim, d_model = H * D, gate rank


def weights(rng, std=0.5, dm=DM, h=H, d=D, rank=RANK):
    hd = h * d
    n = lambda *s: std * rng.standard_normal(s)
    return dict(W_q=n(hd, dm), W_k=n(hd, dm), W_v=n(hd, dm), conv_q=n(hd, 4), conv_k=n(hd, 4),
                conv_v=n(hd, 4), W_down=n(rank, dm), W_up=n(hd, rank), W_beta=n(h, dm),
                W_g=n(hd, dm), W_o=n(dm, hd))


def perm_matrix(perm):
    """P with (x @ P.T)[i] = x[perm[i]], i.e. P[i, perm[i]] = 1."""
    P = np.zeros((len(perm), len(perm)))
    P[np.arange(len(perm)), perm] = 1.0
    return P


IDENTITY_CONV = np.tile([0.0, 0.0, 0.0, 1.0], (H * D, 1))   # tap 3 = current token


# ------------------------------------------------------------------ the pins
def pin_conv_matches_numpy(L):
    """Causal depthwise conv = numpy's full convolution with the reversed taps,
    truncated to the first T outputs."""
    rng = np.random.default_rng(1)
    x, w = rng.standard_normal((17, 5)), rng.standard_normal((5, 4))
    y = L.short_conv(x, w)
    for c in range(5):
        np.testing.assert_allclose(y[:, c], np.convolve(x[:, c], w[c, ::-1])[:17], atol=1e-13)


def pin_conv_impulse_is_causal(L):
    """A unit impulse at t0 excites t0..t0+3 only, with the taps last to first."""
    rng = np.random.default_rng(2)
    w = rng.standard_normal((3, 4))
    x = np.zeros((10, 3))
    x[4, 1] = 1.0
    y = L.short_conv(x, w)
    expect = np.zeros((10, 3))
    for s in range(4):
        expect[4 + s, 1] = w[1, 3 - s]
    np.testing.assert_array_equal(y, expect)


def pin_activations(L):
    x = np.concatenate([np.linspace(-30, 30, 121), [-800.0, 800.0]])
    np.testing.assert_allclose(L.sigmoid(x), expit(x), rtol=1e-15, atol=0)
    np.testing.assert_allclose(L.softplus(x), np.logaddexp(0.0, x), rtol=1e-15, atol=0)
    np.testing.assert_allclose(L.softplus(x) - L.softplus(-x), x, rtol=1e-13, atol=1e-13)
    assert np.all(np.isfinite(L.softplus(x))) and np.all(np.isfinite(L.sigmoid(x)))


def pin_decay_gate_closed_form(L):
    """With W_down x = (1, 0, 0) the gate input is u = W_up[:, 0] for every
    token, and log alpha = -softplus(u) = log sigmoid(-u)."""
    rng = np.random.default_rng(3)
    W = weights(rng)
    x = rng.standard_normal((6, DM))
    x[:, 0] = 1.0
    W["W_down"] = np.zeros((RANK, DM))
    W["W_down"][0, 0] = 1.0
    c = rng.uniform(-4, 4, H * D)
    W["W_up"][:, 0] = c
    p = L.layer_inputs_to_kda(x, W, H, D)
    expect = np.log(expit(-c)).reshape(H, D)
    for t in range(6):
        np.testing.assert_allclose(p["g"][t], expect, rtol=1e-13)
    W["W_down"][:] = 0.0                         # u = 0: alpha = 1/2
    p = L.layer_inputs_to_kda(x, W, H, D)
    np.testing.assert_allclose(p["g"], -np.log(2.0), rtol=1e-15)


def pin_projection_orientation_and_activations(L):
    """W_q = W_v = permutation matrices and identity convs: v = Swish of the
    permuted input, q its per-head L2-normalised version."""
    rng = np.random.default_rng(4)
    W = weights(rng)
    perm_v, perm_q = rng.permutation(DM), rng.permutation(DM)
    W["W_v"], W["W_q"] = perm_matrix(perm_v), perm_matrix(perm_q)
    W["conv_v"], W["conv_q"] = IDENTITY_CONV.copy(), IDENTITY_CONV.copy()
    x = 3.0 * rng.standard_normal((5, DM))
    p = L.layer_inputs_to_kda(x, W, H, D)
    sv = x[:, perm_v] * expit(x[:, perm_v])
    np.testing.assert_allclose(p["v"].reshape(5, DM), sv, rtol=1e-14, atol=1e-15)
    s = (x[:, perm_q] * expit(x[:, perm_q])).reshape(5, H, D)
    q = p["q"]
    ss = (s * s).sum(-1)
    np.testing.assert_allclose((q * q).sum(-1), ss / (ss + 1e-6), rtol=1e-13)
    ratio = q / s                                 # positive and equal within a head
    assert np.all(ratio > 0)
    np.testing.assert_allclose(ratio, ratio[..., :1] * np.ones_like(ratio), rtol=1e-13)


def pin_beta_gate(L):
    """W_beta rows = unit vectors: beta[t, h] = sigmoid(x[t, j_h])."""
    rng = np.random.default_rng(5)
    W = weights(rng)
    j = np.array([5, 2])
    W["W_beta"] = np.zeros((H, DM))
    W["W_beta"][np.arange(H), j] = 1.0
    x = 4.0 * rng.standard_normal((7, DM))
    p = L.layer_inputs_to_kda(x, W, H, D)
    np.testing.assert_allclose(p["beta"], expit(x[:, j]), rtol=1e-15)


def pin_single_token_closed_form(L):
    """T = 1 from the zero state: S_1 = beta k v^T, so o = beta (k . q) v; and
    at the first token only conv tap 3 contributes."""
    rng = np.random.default_rng(6)
    W = weights(rng)
    x = rng.standard_normal((1, 1, DM))
    y, o, parts = L.layer_forward(x, W, H, D)
    p = parts[0]
    kq = (p["k"][0] * p["q"][0]).sum(-1)          # [H]
    np.testing.assert_allclose(o[0, 0], (p["beta"][0] * kq)[:, None] * p["v"][0], rtol=1e-12)
    W2 = dict(W)
    for n in ("conv_q", "conv_k", "conv_v"):
        W2[n] = W[n] * np.array([0.0, 0.0, 0.0, 1.0])
    p2 = L.layer_inputs_to_kda(x[0], W2, H, D)
    for n in ("q", "k", "v"):
        np.testing.assert_array_equal(p2[n], p[n])


def pin_zero_values_give_zero_output(L):
    rng = np.random.default_rng(7)
    W = weights(rng)
    W["W_v"] = np.zeros_like(W["W_v"])
    y, o, _ = L.layer_forward(rng.standard_normal((1, 9, DM)), W, H, D)
    assert np.all(o == 0) and np.all(y == 0)


def pin_output_norm_and_gate(L):
    """W_g = 0 (gate sigmoid(0) = 1/2) and W_o a permutation: after undoing the
    permutation, each head of the layer output is a positive multiple of the
    KDA output with mean square (1/4) ms / (ms + 1e-6), ms = mean square of o."""
    rng = np.random.default_rng(8)
    W = weights(rng)
    W["W_g"] = np.zeros_like(W["W_g"])
    perm = rng.permutation(DM)
    W["W_o"] = perm_matrix(perm)
    y, o, _ = L.layer_forward(rng.standard_normal((1, 11, DM)), W, H, D)
    z = np.empty_like(y[0])
    z[:, perm] = y[0]
    z = z.reshape(11, H, D)
    oh = o[0]
    ms = (oh * oh).mean(-1)
    np.testing.assert_allclose((z * z).mean(-1), 0.25 * ms / (ms + 1e-6), rtol=1e-12)
    ratio = z / oh
    assert np.all(ratio > 0)
    np.testing.assert_allclose(ratio, ratio[..., :1] * np.ones_like(ratio), rtol=1e-12)


def pin_causality(L):
    rng = np.random.default_rng(9)
    W = weights(rng)
    x = rng.standard_normal((1, 12, DM))
    y, _, _ = L.layer_forward(x, W, H, D)
    x2 = x.copy()
    x2[:, 7:] += rng.standard_normal((1, 5, DM))
    y2, _, _ = L.layer_forward(x2, W, H, D)
    np.testing.assert_array_equal(y2[:, :7], y[:, :7])
    assert np.max(np.abs(y2[:, 7] - y[:, 7])) > 1e-6


def pin_sequences_independent(L):
    rng = np.random.default_rng(10)
    W = weights(rng)
    x = rng.standard_normal((2, 6, DM))
    y, o, _ = L.layer_forward(x, W, H, D)
    for b in range(2):
        yb, ob, _ = L.layer_forward(x[b:b + 1], W, H, D)
        np.testing.assert_array_equal(yb[0], y[b])
        np.testing.assert_array_equal(ob[0], o[b])


PINS = [pin_conv_matches_numpy, pin_conv_impulse_is_causal, pin_activations,
        pin_decay_gate_closed_form, pin_projection_orientation_and_activations, pin_beta_gate,
        pin_single_token_closed_form, pin_zero_values_give_zero_output, pin_output_norm_and_gate,
        pin_causality, pin_sequences_independent]


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_layer_oracle_pin(pin):
    pin(kda_layer_ref)


# ------------------------------------------------------------------ mutations
MUTATIONS = {
    "conv_taps_reversed": ("shift = K - 1 - j", "shift = j"),
    "conv_acausal": ("y[shift:] += w[:, j][None, :] * x[:T - shift]",
                     "y[:T - shift] += w[:, j][None, :] * x[shift:]"),
    "no_swish_on_v": ('v = swish(short_conv(vp, Wf["conv_v"]))', 'v = short_conv(vp, Wf["conv_v"])'),
    "no_l2norm_on_q": ('q = l2norm_heads(swish(short_conv(qp, Wf["conv_q"])), H, d)',
                       'q = swish(short_conv(qp, Wf["conv_q"]))'),
    "rmsnorm_with_sum": (".mean(-1, keepdims=True) + EPS_RMS", ".sum(-1, keepdims=True) + EPS_RMS"),
    "decay_sign": ('g = -softplus(', 'g = softplus('),
    "gate_without_sigmoid": ('* sigmoid(p["gate"])', '* p["gate"]'),
    "projection_transposed": ('vp = x @ Wf["W_v"].T', 'vp = x @ Wf["W_v"]'),
    "beta_without_sigmoid": ('beta = sigmoid(x @ Wf["W_beta"].T)', 'beta = x @ Wf["W_beta"].T'),
    "softplus_wrong_branch": ("np.maximum(x, 0.0) + np.log1p(np.exp(-np.abs(x)))",
                              "np.maximum(x, 0.0) + np.log1p(np.exp(np.abs(x)))"),
}


def mutant(kind):
    old, new = MUTATIONS[kind]
    src = open(kda_layer_ref.__file__).read()
    assert src.count(old) == 1, f"mutation site for {kind} not found exactly once"
    mod = types.ModuleType("oracle._layer_mutant")
    mod.__package__ = "oracle"
    mod.__file__ = kda_layer_ref.__file__
    exec(compile(src.replace(old, new), mod.__file__, "exec"), mod.__dict__)
    return mod


@pytest.mark.filterwarnings("ignore::RuntimeWarning")
@pytest.mark.parametrize("kind", sorted(MUTATIONS))
def test_layer_pins_catch_planted_mistakes(kind):
    L = mutant(kind)
    failed = []
    for pin in PINS:
        try:
            pin(L)
        except Exception:                          # an assertion or a shape error
            failed.append(pin.__name__)
    assert failed, f"no pin caught {kind}"
    assert "oracle._layer_mutant" not in sys.modules
