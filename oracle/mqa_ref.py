"""CPU oracle for the full-attention decode step KDA is compared against.
TEST INFRASTRUCTURE: only the test suite, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module.  It shares no code
with the GPU library.

Page "Kimi K3论文：Kimi Linear", section 5: the full-attention layers of the
hybrid are MLA with no position encoding, which at inference reduces to MQA
over the layer's per-token latent.  Section 7 compares decode time per output
token at 1M context against a full-MLA model.  The decode step of such a layer
is, for every query head h of sequence b (the latent c_t serving as key and
value):

    o[b, h] = sum_t softmax_t(scale * q[b, h] . c[b, t]) c[b, t]

:func:`decode` evaluates exactly that in fp64: all scores of a head first,
then the max-shifted exponentials, their sum, and the weighted sum of the
latents.  The weighted sum runs over blocks of tokens only to bound memory; no
online rescaling is involved (the shift is the global maximum).
"""
from __future__ import annotations

import numpy as np


def _f64(x):
    if hasattr(x, "detach"):
        x = x.detach().to("cpu").double().numpy()
    return np.asarray(x, dtype=np.float64)


def decode(q, cache, scale, heads=None, block=65536):
    """q [B, H, D], cache [B, T, D] (any float dtype, upcast exactly), returns
    o [B, H', D] in fp64 for the heads listed in ``heads`` (default all)."""
    q = _f64(q)
    B, H, D = q.shape
    T = cache.shape[1]
    hs = list(range(H)) if heads is None else list(heads)
    out = np.zeros((B, len(hs), D))
    for b in range(B):
        qb = q[b, hs]                                    # [H', D]
        scores = np.empty((len(hs), T))
        for t0 in range(0, T, block):
            cb = _f64(cache[b, t0:t0 + block])
            scores[:, t0:t0 + cb.shape[0]] = scale * (qb @ cb.T)
        m = scores.max(axis=1, keepdims=True)
        p = np.exp(scores - m)
        denom = p.sum(axis=1)
        acc = np.zeros((len(hs), D))
        for t0 in range(0, T, block):
            cb = _f64(cache[b, t0:t0 + block])
            acc += p[:, t0:t0 + cb.shape[0]] @ cb
        out[b] = acc / denom[:, None]
    return out
