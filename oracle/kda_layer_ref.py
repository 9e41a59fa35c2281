"""CPU oracle for one KDA token-mixing layer (fp64).  TEST INFRASTRUCTURE.

Only the test suite, the smoke check and the CPU-baseline leg of the benchmark
may import this module; it shares no code with the GPU library.

The layer follows page "Kimi K3论文：Kimi Linear", section 3 (input
parameterisation and output path), around the KDA recurrence of eq. (1):

  q, k = L2Norm(Swish(ShortConv(W_q x))), L2Norm(Swish(ShortConv(W_k x)))
  v    = Swish(ShortConv(W_v x))
  g    = log alpha = -softplus(W_up (W_down x))        (alpha = exp(-softplus(.)))
  beta = Sigmoid(W_beta x)
  o    = KDA(q, k, v, g, beta)                          (per head, S0 = 0)
  y    = W_o ( RMSNorm(o per head) * Sigmoid(W_g x) )

Readings of what the page leaves open (each also stated where it is used):
  * the decay function f is exp(-softplus(.)) (the workload recipe fixes it);
  * ShortConv is a causal depthwise convolution with 4 taps per channel, zero
    left padding and no bias: y_t[c] = sum_{j=0..3} w[c, j] x_{t-3+j}[c];
  * Swish(x) = x * sigmoid(x); L2Norm(x) = x / sqrt(sum x^2 + 1e-6) over the
    128 channels of a head; RMSNorm(x) = x / sqrt(mean x^2 + 1e-6) over a
    head, with no learned gain (random-init weights carry none);
  * the output gate is a full-rank W_g (d_model x H*128) followed by sigmoid;
  * biases are zero; weight matrices are stored [out_features, in_features].
Everything is computed in fp64 from the given (bf16-exact) values, with no
intermediate rounding.
"""
from __future__ import annotations

import numpy as np

from . import kda_ref

EPS_L2 = 1e-6
EPS_RMS = 1e-6


def _f64(x):
    if hasattr(x, "detach"):
        x = x.detach().to("cpu").double().numpy()
    return np.asarray(x, dtype=np.float64)


def sigmoid(x):
    """1 / (1 + e^-x), evaluated without overflow for either sign."""
    x = np.asarray(x, np.float64)
    out = np.empty_like(x)
    pos = x >= 0
    out[pos] = 1.0 / (1.0 + np.exp(-x[pos]))
    e = np.exp(x[~pos])
    out[~pos] = e / (1.0 + e)
    return out


def softplus(x):
    """log(1 + e^x) = max(x, 0) + log1p(e^-|x|)."""
    x = np.asarray(x, np.float64)
    return np.maximum(x, 0.0) + np.log1p(np.exp(-np.abs(x)))


def swish(x):
    return x * sigmoid(x)


def short_conv(x, w):
    """Causal depthwise convolution.  x [T, C], w [C, K] -> [T, C] with
    y_t[c] = sum_j w[c, j] * x_{t-(K-1)+j}[c], x_s = 0 for s < 0."""
    T, Cn = x.shape
    K = w.shape[1]
    y = np.zeros_like(x)
    for j in range(K):
        shift = K - 1 - j
        if shift >= T:
            continue
        y[shift:] += w[:, j][None, :] * x[:T - shift]
    return y


def l2norm_heads(x, H, d):
    """Per-head L2 normalisation of [T, H*d] (eps 1e-6 inside the root)."""
    T = x.shape[0]
    xh = x.reshape(T, H, d)
    return (xh / np.sqrt((xh * xh).sum(-1, keepdims=True) + EPS_L2)).reshape(T, H * d)


def rmsnorm_heads(x, H, d):
    T = x.shape[0]
    xh = x.reshape(T, H, d)
    return (xh / np.sqrt((xh * xh).mean(-1, keepdims=True) + EPS_RMS)).reshape(T, H * d)


def layer_inputs_to_kda(x, W, H, d=128):
    """The projections, ShortConv, activations and gates of the layer for ONE
    sequence x [T, d_model].  Returns dict q, k, v [T, H, d], g [T, H, d],
    beta [T, H], gate [T, H*d] (pre-sigmoid)."""
    x = _f64(x)
    T = x.shape[0]
    Wf = {n: _f64(w) for n, w in W.items()}
    qp = x @ Wf["W_q"].T
    kp = x @ Wf["W_k"].T
    vp = x @ Wf["W_v"].T
    q = l2norm_heads(swish(short_conv(qp, Wf["conv_q"])), H, d)
    k = l2norm_heads(swish(short_conv(kp, Wf["conv_k"])), H, d)
    v = swish(short_conv(vp, Wf["conv_v"]))
    g = -softplus((x @ Wf["W_down"].T) @ Wf["W_up"].T)
    beta = sigmoid(x @ Wf["W_beta"].T)
    gate = x @ Wf["W_g"].T
    sh = lambda a: a.reshape(T, H, d)
    return dict(q=sh(q), k=sh(k), v=sh(v), g=sh(g), beta=beta, gate=gate)


def layer_forward(x, W, H, d=128):
    """Full layer for x [B, T, d_model] (B independent sequences).  Returns
    (y [B, T, d_model], o [B, T, H, d] (the KDA output), per-sequence dicts of
    the KDA inputs)."""
    x = _f64(x)
    B, T, _ = x.shape
    ys, os_, parts = [], [], []
    for b in range(B):
        p = layer_inputs_to_kda(x[b], W, H, d)
        o, _ = kda_ref.recurrent(p["q"][None], p["k"][None], p["v"][None], p["g"][None],
                                 p["beta"][None], None)
        o = o[0]                                           # [T, H, d]
        z = rmsnorm_heads(o.reshape(T, H * d), H, d) * sigmoid(p["gate"])
        ys.append(z @ _f64(W["W_o"]).T)
        os_.append(o)
        parts.append(p)
    return np.stack(ys), np.stack(os_), parts
