"""Seeded synthetic inputs for the KDA workloads (shared by tests and bench).

This module draws random numbers and casts them; it holds none of the KDA
arithmetic.  The draws follow the workload recipes (shapes, distributions,
dtypes); rounding to bf16 is round-to-nearest-even (torch's cast), and the
oracle consumes exactly the rounded values.

Prefill draws: ``numpy.random.default_rng(seed)``, in the order q, k, v, g,
beta, S0, each ``[B, T, H, .]`` in C order, as fp32:
  q, k ~ N(0, 1), then divided by their L2 norm per (token, head);
  v ~ N(0, 1);
  g = -g_scale * softplus(N(0, 1))  (log of the per-channel forget gate; with
      gate="head" one draw per (token, head), shape [B, T, H]: the Gated
      DeltaNet gate; with gate="none" no draw and g = None: DeltaNet);
  beta = sigmoid(N(0, 1));
  S0 ~ N(0, s0_std^2) if s0_std > 0 else None.
Decode draws (per step, one token per (sequence, head)) use a torch generator
on the target device so that 1000 steps of tokens can be drawn quickly:
  q, k ~ N(0,1) L2-normalised, v ~ N(0,1), beta = sigmoid(N(0,1)),
  alpha ~ U[0.9, 1] and g = log(alpha); state S ~ N(0, 0.02^2).
"""
from __future__ import annotations

import numpy as np

D = 128

# The five workloads: name -> recipe.  Sizes are the full ones.
PREFILL_CONFIGS = {
    "c1_fp32_T256": dict(B=1, T=256, H=1, dtype="float32", g_scale=0.1, s0_std=0.0, seed=1),
    "c2_bf16_B8_H16_T4096": dict(B=8, T=4096, H=16, dtype="bfloat16", g_scale=0.05, s0_std=0.0, seed=2),
    "c3_bf16_B1_H32_T65536": dict(B=1, T=65536, H=32, dtype="bfloat16", g_scale=0.05, s0_std=0.02, seed=3),
    # the B = 8, H = 16, T = 4096 prefill with the other two gates of the family
    "c2_gdn_bf16_B8_H16_T4096": dict(B=8, T=4096, H=16, dtype="bfloat16", g_scale=0.05, s0_std=0.0, seed=2,
                                     gate="head"),
    "c2_deltanet_bf16_B8_H16_T4096": dict(B=8, T=4096, H=16, dtype="bfloat16", g_scale=0.05, s0_std=0.0,
                                          seed=2, gate="none"),
}
DECODE_CONFIG = dict(N=256, H=32, steps=1000, dtype="bfloat16", s_std=0.02, seed=4)
LAYER_CONFIG = dict(B=1, T=32768, d_model=2048, H=16, dtype="bfloat16", w_std=0.02, seed=5)


def _torch_dtype(name):
    import torch
    return {"float32": torch.float32, "bfloat16": torch.bfloat16}[name]


def _l2n(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def _softplus(x):
    return np.logaddexp(np.float32(0.0), x).astype(np.float32)


def _sigmoid(x):
    return (1.0 / (1.0 + np.exp(-x))).astype(np.float32)


def prefill_inputs(B, T, H, dtype="bfloat16", g_scale=0.05, s0_std=0.0, seed=0, d=D, gate="channel"):
    """Returns a dict of CPU torch tensors q, k, v, g, beta (and S0 or None).
    gate: "channel" (g [B, T, H, d]), "head" (g [B, T, H]) or "none" (g None)."""
    import torch
    rng = np.random.default_rng(seed)
    shp = (B, T, H, d)
    q = _l2n(rng.standard_normal(shp, dtype=np.float32))
    k = _l2n(rng.standard_normal(shp, dtype=np.float32))
    v = rng.standard_normal(shp, dtype=np.float32)
    gshp = {"channel": shp, "head": (B, T, H), "none": None}[gate]
    g = None if gshp is None else (-np.float32(g_scale)) * _softplus(rng.standard_normal(gshp, dtype=np.float32))
    beta = _sigmoid(rng.standard_normal((B, T, H), dtype=np.float32))
    S0 = None
    if s0_std > 0:
        S0 = torch.from_numpy(np.float32(s0_std) * rng.standard_normal((B, H, d, d), dtype=np.float32))
    td = _torch_dtype(dtype)
    cast = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(td)
    return dict(q=cast(q), k=cast(k), v=cast(v),
                g=None if g is None else torch.from_numpy(np.ascontiguousarray(g)),
                beta=cast(beta), S0=S0)


def grad_inputs(B, T, H, dtype="bfloat16", ds_std=0.0, seed=0, d=D):
    """Incoming gradients for the backward pass: dO ~ N(0, 1) in `dtype`
    [B, T, H, d] and dS_T ~ N(0, ds_std^2) fp32 [B, H, d, d] (None when
    ds_std is 0), from a generator of their own (seed, 1)."""
    import torch
    rng = np.random.default_rng([seed, 1])
    dO = torch.from_numpy(rng.standard_normal((B, T, H, d), dtype=np.float32)).to(_torch_dtype(dtype))
    dST = None
    if ds_std > 0:
        dST = torch.from_numpy(np.float32(ds_std) * rng.standard_normal((B, H, d, d), dtype=np.float32))
    return dict(dO=dO, dS_T=dST)


# General diagonal-plus-low-rank transition at the B = 8, H = 16, T = 4096 shape
DPLR_CONFIG = dict(B=8, T=4096, H=16, dtype="bfloat16", g_scale=0.05, s0_std=0.0, seed=7)


def dplr_inputs(B, T, H, dtype="bfloat16", g_scale=0.05, s0_std=0.0, seed=0, d=D):
    """Inputs of the DPLR recurrence S_t = (Diag(e^{g_t}) - a_t b_t^T) S_{t-1} +
    k_t v_t^T, o_t = S_t^T q_t.  ``numpy.random.default_rng(seed)``, drawn in
    the order q, k, v, g, beta, ka, kb, S0: q, k, v, g, beta as for the prefill
    (q, k L2-normalised, g = -g_scale softplus(N(0,1)) per channel, beta =
    sigmoid(N(0,1))); ka, kb ~ N(0,1) L2-normalised, independent of k;
    a = beta * ka and b = e^{g} * kb -- the shape of KDA's a and b (beta k and
    alpha * k) with the two vectors no longer tied to each other or to k.
    Returns a dict of CPU tensors q, k, v, a, b (dtype), g (fp32), S0 or None."""
    import torch
    rng = np.random.default_rng(seed)
    shp = (B, T, H, d)
    q = _l2n(rng.standard_normal(shp, dtype=np.float32))
    k = _l2n(rng.standard_normal(shp, dtype=np.float32))
    v = rng.standard_normal(shp, dtype=np.float32)
    g = (-np.float32(g_scale)) * _softplus(rng.standard_normal(shp, dtype=np.float32))
    beta = _sigmoid(rng.standard_normal((B, T, H), dtype=np.float32))
    ka = _l2n(rng.standard_normal(shp, dtype=np.float32))
    kb = _l2n(rng.standard_normal(shp, dtype=np.float32))
    S0 = None
    if s0_std > 0:
        S0 = torch.from_numpy(np.float32(s0_std) * rng.standard_normal((B, H, d, d), dtype=np.float32))
    td = _torch_dtype(dtype)
    cast = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(td)
    return dict(q=cast(q), k=cast(k), v=cast(v), a=cast(beta[..., None] * ka), b=cast(np.exp(g) * kb),
                g=torch.from_numpy(np.ascontiguousarray(g)), S0=S0)


MQA_CONFIG = dict(B=1, T=1 << 20, H=32, D=512, seed=6)


def mqa_inputs(B, T, H, D=512, seed=0, device="cpu"):
    """Query heads and latent cache of a full-attention decode step: q [B, H, D]
    and cache [B, T, D], both N(0, 1) rounded to bf16 (torch generator on
    `device`, so a 1M-token cache is drawn where it is used)."""
    import torch
    gen = torch.Generator(device=device).manual_seed(seed)
    q = torch.randn((B, H, D), generator=gen, device=device, dtype=torch.float32).to(torch.bfloat16)
    cache = torch.randn((B, T, D), generator=gen, device=device, dtype=torch.float32).to(torch.bfloat16)
    return q, cache


def prefill_config(name, **override):
    """Inputs of a named prefill workload; keyword overrides (e.g. T=...)."""
    cfg = dict(PREFILL_CONFIGS[name])
    cfg.update(override)
    return prefill_inputs(**cfg)


def decode_state(N, H, s_std=0.02, seed=0, device="cpu", d=D):
    import torch
    gen = torch.Generator(device=device).manual_seed(seed)
    return s_std * torch.randn((N, H, d, d), generator=gen, device=device, dtype=torch.float32)


def decode_tokens(N, H, steps, dtype="bfloat16", seed=0, device="cpu", d=D, gate="channel"):
    """Tokens for ``steps`` decode steps: dict of tensors with a leading step
    axis, q/k/v [steps, N, H, d], g [steps, N, H, d] fp32 (gate="head": [steps,
    N, H]; gate="none": None), beta [steps, N, H]."""
    import torch
    gen = torch.Generator(device=device).manual_seed(seed + 1)
    td = _torch_dtype(dtype)
    f32 = torch.float32

    def l2n(x):
        return x / torch.linalg.vector_norm(x, dim=-1, keepdim=True)

    q = l2n(torch.randn((steps, N, H, d), generator=gen, device=device, dtype=f32)).to(td)
    k = l2n(torch.randn((steps, N, H, d), generator=gen, device=device, dtype=f32)).to(td)
    v = torch.randn((steps, N, H, d), generator=gen, device=device, dtype=f32).to(td)
    beta = torch.sigmoid(torch.randn((steps, N, H), generator=gen, device=device, dtype=f32)).to(td)
    gshp = {"channel": (steps, N, H, d), "head": (steps, N, H), "none": None}[gate]
    g = None
    if gshp is not None:
        alpha = 0.9 + 0.1 * torch.rand(gshp, generator=gen, device=device, dtype=f32)
        g = torch.log(alpha)
    return dict(q=q, k=k, v=v, g=g, beta=beta)


def layer_inputs(B=1, T=32768, d_model=2048, H=16, dtype="bfloat16", w_std=0.02, seed=5,
                 d=D, conv_taps=4, gate_rank=D):
    """Input x and random-init weights of one KDA token-mixing layer.  Weight
    matrices are stored [out_features, in_features]; draws in the order x, W_q,
    W_k, W_v, conv_q, conv_k, conv_v, W_down, W_up, W_beta, W_g, W_o."""
    import torch
    rng = np.random.default_rng(seed)
    td = _torch_dtype(dtype)
    hd = H * d
    nrm = lambda *s: rng.standard_normal(s, dtype=np.float32)
    x = nrm(B, T, d_model)
    w = {}
    for name, shape in (("W_q", (hd, d_model)), ("W_k", (hd, d_model)), ("W_v", (hd, d_model)),
                        ("conv_q", (hd, conv_taps)), ("conv_k", (hd, conv_taps)),
                        ("conv_v", (hd, conv_taps)), ("W_down", (gate_rank, d_model)),
                        ("W_up", (hd, gate_rank)), ("W_beta", (H, d_model)),
                        ("W_g", (hd, d_model)), ("W_o", (d_model, hd))):
        w[name] = torch.from_numpy(np.float32(w_std) * nrm(*shape)).to(td)
    return dict(x=torch.from_numpy(x).to(td), **w)
