"""libkda Python binding: Kimi Delta Attention kernels for MI355X (gfx950).

``chunk_fwd`` (chunkwise prefill), ``chunk_bwd`` (its backward pass),
``recurrent_step`` (decode) and ``layer_fwd`` (one token-mixing layer) take
torch tensors on the GPU and call the C ABI of ``libkda.so`` on the current
stream.
torch is used for device memory and streams only.
"""
from __future__ import annotations

import ctypes

from ._binding import (KDA_BF16, KDA_F32, KDA_GATE_CHANNEL, KDA_GATE_HEAD,  # noqa: F401
                       KDA_GATE_NONE, LAYER_REGIONS, KDAError, lib, status_string, version, _check)

__all__ = ["chunk_fwd", "chunk_fwd_varlen", "chunk_bwd", "bwd_workspace_size", "dplr_chunk_fwd", "recurrent_steps",
           "dplr_workspace_size", "recurrent_step", "workspace_size", "scan_workspace_bytes",
           "layer_fwd", "layer_workspace_layout", "LAYER_WEIGHTS", "mqa_decode", "release_workspaces",
           "status_string", "version", "KDAError",
           "KDA_F32", "KDA_BF16", "lib"]


def _dtype_code(t):
    import torch
    if t.dtype == torch.bfloat16:
        return KDA_BF16
    if t.dtype == torch.float32:
        return KDA_F32
    raise TypeError(f"unsupported dtype {t.dtype}: use torch.float32 or torch.bfloat16")


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(device):
    import torch
    return torch.cuda.current_stream(device).cuda_stream


def _need(t, name, dtype, shape, device):
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


_ws_cache = {}


def workspace_size(B, T, H, dtype_code, d=128):
    """Workspace bytes kda_chunk_fwd wants for its fastest schedule (0: none)."""
    return int(lib().kda_chunk_fwd_workspace_size(B, T, H, d, d, dtype_code))


def scan_workspace_bytes(B, T, H, d=128):
    """Workspace that selects the two-kernel schedule with a one-pass state
    scan for any bf16 shape (:func:`workspace_size` adds, for 16 heads or
    fewer, the buffers of the segmented scan); asked of the library."""
    return int(lib().kda_chunk_fwd_scan_workspace_size(B, T, H, d, d, KDA_BF16))


def _workspace(device, nbytes):
    """The "auto" workspace: at most one buffer per (device, stream), so calls
    on different streams never share scratch memory.  A cached buffer is
    reused when it holds the request and is at most twice its size; otherwise
    it is replaced by one of the requested size, so the cache never keeps much
    more than the last call needed.  It is allocated while that stream is
    current, so torch's allocator orders its reuse after the stream's pending
    work when it is replaced.  :func:`release_workspaces` drops the cache."""
    import torch
    if nbytes <= 0:
        return None
    key = (torch.device(device), _stream(device))
    buf = _ws_cache.get(key)
    if buf is None or buf.numel() < nbytes or buf.numel() > 2 * nbytes:
        _ws_cache.pop(key, None)
        buf = torch.empty(nbytes, dtype=torch.uint8, device=device)
        _ws_cache[key] = buf
    return buf


def release_workspaces():
    """Drop every cached "auto" workspace (their memory returns to torch's
    allocator once the streams' pending work no longer uses it)."""
    _ws_cache.clear()


def _gate(log_alpha, per_channel_dim):
    """Gate kind from the shape of log_alpha: None -> no decay (DeltaNet), one
    value per head -> Gated DeltaNet, one per channel -> KDA."""
    if log_alpha is None:
        return KDA_GATE_NONE
    return KDA_GATE_CHANNEL if log_alpha.dim() == per_channel_dim else KDA_GATE_HEAD


def chunk_fwd(q, k, v, log_alpha, beta, S0=None, *, out=None, S_T=None,
              return_state: bool = True, workspace="auto"):
    """Chunked KDA prefill.  q, k, v: [B, T, H, 128] (fp32 or bf16); log_alpha:
    [B, T, H, 128] fp32 (KDA), [B, T, H] fp32 (one decay per head: Gated
    DeltaNet) or None (no decay: DeltaNet); beta: [B, T, H] (same dtype as q);
    S0: [B, H, 128, 128] fp32 or None.  ``workspace``: "auto" (the size the
    library asks for, cached per device), None (fused single-kernel schedule)
    or a uint8 device tensor.  Returns ``(o, S_T)`` (``S_T`` is None if not
    requested)."""
    import torch
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    dev, dt = q.device, q.dtype
    code = _dtype_code(q)
    for t, n, shp in ((k, "k", q.shape), (v, "v", (B, T, H, dv)), (beta, "beta", (B, T, H))):
        _need(t, n, dt, shp, dev)
    gate = _gate(log_alpha, 4)
    if gate != KDA_GATE_NONE:
        _need(log_alpha, "log_alpha", torch.float32, q.shape if gate == KDA_GATE_CHANNEL else (B, T, H), dev)
    _need(q, "q", dt, q.shape, dev)
    if S0 is not None:
        _need(S0, "S0", torch.float32, (B, H, dk, dv), dev)
    if out is None:
        out = torch.empty((B, T, H, dv), dtype=dt, device=dev)
    else:
        _need(out, "out", dt, (B, T, H, dv), dev)
    if S_T is None and return_state:
        S_T = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
    elif S_T is not None:
        _need(S_T, "S_T", torch.float32, (B, H, dk, dv), dev)
    if isinstance(workspace, str):
        if workspace != "auto":
            raise ValueError("workspace must be 'auto', None or a tensor")
        workspace = _workspace(dev, workspace_size(B, T, H, code, dk))
    ws_ptr, ws_bytes = None, 0
    if workspace is not None:
        if workspace.device != dev or workspace.dtype != torch.uint8:
            raise ValueError("workspace must be a uint8 tensor on the same device")
        ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel()
    st = lib().kda_chunk_fwd_gated(_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), gate, _ptr(beta),
                                   _ptr(S0), _ptr(out), _ptr(S_T), B, T, H, dk, dv, code,
                                   ws_ptr, ws_bytes, _stream(dev))
    _check("kda_chunk_fwd_gated", st)
    return out, S_T


def chunk_fwd_varlen(q, k, v, log_alpha, beta, cu_seqlens, S0=None, *, out=None, S_T=None,
                     return_state: bool = True):
    """Chunked prefill over sequences packed along one token axis.  q, k, v:
    [total, H, 128]; log_alpha: [total, H, 128] / [total, H] fp32 or None (gate
    as for chunk_fwd); beta: [total, H]; cu_seqlens: int32 device tensor
    [num_seqs + 1] of sequence offsets; S0: [num_seqs, H, 128, 128] fp32 or
    None.  Returns ``(o, S_T)``; S_T is [num_seqs, H, 128, 128]."""
    import torch
    total, H, dk = q.shape
    dv = v.shape[-1]
    dev, dt = q.device, q.dtype
    code = _dtype_code(q)
    ns = cu_seqlens.numel() - 1
    _need(cu_seqlens, "cu_seqlens", torch.int32, (ns + 1,), dev)
    for t, n, shp in ((k, "k", q.shape), (v, "v", (total, H, dv)), (beta, "beta", (total, H))):
        _need(t, n, dt, shp, dev)
    gate = _gate(log_alpha, 3)
    if gate != KDA_GATE_NONE:
        _need(log_alpha, "log_alpha", torch.float32, q.shape if gate == KDA_GATE_CHANNEL else (total, H), dev)
    if S0 is not None:
        _need(S0, "S0", torch.float32, (ns, H, dk, dv), dev)
    if out is None:
        out = torch.empty((total, H, dv), dtype=dt, device=dev)
    else:
        _need(out, "out", dt, (total, H, dv), dev)
    if S_T is None and return_state:
        S_T = torch.empty((ns, H, dk, dv), dtype=torch.float32, device=dev)
    elif S_T is not None:
        _need(S_T, "S_T", torch.float32, (ns, H, dk, dv), dev)
    st = lib().kda_chunk_fwd_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), gate, _ptr(beta),
                                    _ptr(cu_seqlens), ns, _ptr(S0), _ptr(out), _ptr(S_T),
                                    total, H, dk, dv, code, _stream(dev))
    _check("kda_chunk_fwd_varlen", st)
    return out, S_T


def mqa_decode(q, cache, scale, *, out=None, workspace=None):
    """Full-attention decode step (MQA over a shared latent: the inference form
    of a NoPE MLA layer).  q [B, H, 512] bf16, cache [B, T, 512] bf16; returns
    o [B, H, 512] bf16 = softmax(scale q c^T) c per head."""
    import torch
    B, H, D = q.shape
    T = cache.shape[1]
    dev = q.device
    _need(q, "q", torch.bfloat16, (B, H, D), dev)
    _need(cache, "cache", torch.bfloat16, (B, T, D), dev)
    if out is None:
        out = torch.empty((B, H, D), dtype=torch.bfloat16, device=dev)
    else:
        _need(out, "out", torch.bfloat16, (B, H, D), dev)
    if workspace is None:
        workspace = _workspace(dev, int(lib().kda_mqa_decode_workspace_size(B, T, H, D)))
    ws_ptr = None if workspace is None else workspace.data_ptr()
    ws_bytes = 0 if workspace is None else workspace.numel()
    st = lib().kda_mqa_decode(_ptr(q), _ptr(cache), _ptr(out), B, T, H, D, float(scale),
                              ws_ptr, ws_bytes, _stream(dev))
    _check("kda_mqa_decode", st)
    return out


def dplr_workspace_size(B, T, H, d=128):
    """Workspace bytes kda_dplr_chunk_fwd needs (bf16)."""
    return int(lib().kda_dplr_chunk_fwd_workspace_size(B, T, H, d, d, KDA_BF16))


def dplr_chunk_fwd(q, k, v, a, b, log_alpha, S0=None, *, out=None, S_T=None, return_state: bool = True,
                   workspace="auto"):
    """General diagonal-plus-low-rank recurrence S_t = (Diag(e^{log_alpha_t}) -
    a_t b_t^T) S_{t-1} + k_t v_t^T, o_t = S_t^T q_t (bf16 only).  q, k, a, b, v:
    [B, T, H, 128] bf16; log_alpha [B, T, H, 128] fp32; S0 [B, H, 128, 128] fp32
    or None.  ``workspace``: "auto" (cached per device) or a uint8 device tensor
    of at least :func:`dplr_workspace_size` bytes.  Returns (o, S_T)."""
    import torch
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    dev, dt = q.device, q.dtype
    code = _dtype_code(q)
    for t, n in ((k, "k"), (a, "a"), (b, "b")):
        _need(t, n, dt, q.shape, dev)
    _need(v, "v", dt, (B, T, H, dv), dev)
    _need(log_alpha, "log_alpha", torch.float32, q.shape, dev)
    if S0 is not None:
        _need(S0, "S0", torch.float32, (B, H, dk, dv), dev)
    if out is None:
        out = torch.empty((B, T, H, dv), dtype=dt, device=dev)
    else:
        _need(out, "out", dt, (B, T, H, dv), dev)
    if S_T is None and return_state:
        S_T = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
    elif S_T is not None:
        _need(S_T, "S_T", torch.float32, (B, H, dk, dv), dev)
    if isinstance(workspace, str):
        if workspace != "auto":
            raise ValueError("workspace must be 'auto' or a tensor")
        workspace = _workspace(dev, dplr_workspace_size(B, T, H, dk))
    ws_ptr, ws_bytes = None, 0
    if workspace is not None:
        if workspace.device != dev or workspace.dtype != torch.uint8:
            raise ValueError("workspace must be a uint8 tensor on the same device")
        ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel()
    st = lib().kda_dplr_chunk_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(b), _ptr(log_alpha), _ptr(S0),
                                  _ptr(out), _ptr(S_T), B, T, H, dk, dv, code, ws_ptr, ws_bytes, _stream(dev))
    _check("kda_dplr_chunk_fwd", st)
    return out, S_T


def bwd_workspace_size(B, T, H, d=128):
    """Workspace bytes kda_chunk_bwd needs (bf16)."""
    return int(lib().kda_chunk_bwd_workspace_size(B, T, H, d, d, KDA_BF16))


def chunk_bwd(q, k, v, log_alpha, beta, S0, grad_o, grad_S_T=None, *, workspace="auto",
              grad_S0: bool = True):
    """Backward pass of :func:`chunk_fwd` (bf16 only).  Inputs as for chunk_fwd
    plus grad_o [B, T, H, 128] bf16 and grad_S_T [B, H, 128, 128] fp32 (None:
    zero).  ``workspace``: "auto" (cached per device) or a uint8 device tensor
    of at least :func:`bwd_workspace_size` bytes.  Returns ``(dq, dk, dv,
    dlog_alpha, dbeta, dS0)``; dS0 is None when ``grad_S0`` is false.  The
    gate follows log_alpha's shape as in chunk_fwd: [B, T, H, 128] (KDA),
    [B, T, H] (Gated DeltaNet: dlog_alpha [B, T, H]) or None (DeltaNet:
    dlog_alpha None)."""
    import torch
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    dev, dt = q.device, q.dtype
    code = _dtype_code(q)
    for t, n, shp in ((k, "k", q.shape), (v, "v", (B, T, H, dv)), (beta, "beta", (B, T, H)),
                      (grad_o, "grad_o", (B, T, H, dv))):
        _need(t, n, dt, shp, dev)
    gate = _gate(log_alpha, 4)
    if gate != KDA_GATE_NONE:
        _need(log_alpha, "log_alpha", torch.float32, q.shape if gate == KDA_GATE_CHANNEL else (B, T, H), dev)
    for t, n in ((S0, "S0"), (grad_S_T, "grad_S_T")):
        if t is not None:
            _need(t, n, torch.float32, (B, H, dk, dv), dev)
    out = [torch.empty_like(q), torch.empty_like(k), torch.empty_like(v),
           None if log_alpha is None else torch.empty_like(log_alpha), torch.empty_like(beta)]
    dS0 = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev) if grad_S0 else None
    if isinstance(workspace, str):
        if workspace != "auto":
            raise ValueError("workspace must be 'auto' or a tensor")
        workspace = _workspace(dev, bwd_workspace_size(B, T, H, dk))
    ws_ptr, ws_bytes = None, 0
    if workspace is not None:
        if workspace.device != dev or workspace.dtype != torch.uint8:
            raise ValueError("workspace must be a uint8 tensor on the same device")
        ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel()
    st = lib().kda_chunk_bwd_gated(_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), gate, _ptr(beta), _ptr(S0),
                                   _ptr(grad_o), _ptr(grad_S_T), *(_ptr(x) for x in out), _ptr(dS0),
                                   B, T, H, dk, dv, code, ws_ptr, ws_bytes, _stream(dev))
    _check("kda_chunk_bwd_gated", st)
    return (*out, dS0)


def recurrent_step(q, k, v, log_alpha, beta, S, *, out=None):
    """One KDA decode step, state updated in place.  q, k, v: [N, H, 128];
    log_alpha: [N, H, 128] fp32 (KDA), [N, H] fp32 (Gated DeltaNet) or None
    (DeltaNet); beta: [N, H]; S: [N, H, 128, 128] fp32.  Returns o [N, H, 128]."""
    import torch
    N, H, dk = q.shape
    dv = v.shape[-1]
    dev, dt = q.device, q.dtype
    code = _dtype_code(q)
    for t, n, shp in ((k, "k", q.shape), (v, "v", (N, H, dv)), (beta, "beta", (N, H))):
        _need(t, n, dt, shp, dev)
    gate = _gate(log_alpha, 3)
    if gate != KDA_GATE_NONE:
        _need(log_alpha, "log_alpha", torch.float32, q.shape if gate == KDA_GATE_CHANNEL else (N, H), dev)
    _need(S, "S", torch.float32, (N, H, dk, dv), dev)
    if out is None:
        out = torch.empty((N, H, dv), dtype=dt, device=dev)
    else:
        _need(out, "out", dt, (N, H, dv), dev)
    st = lib().kda_recurrent_step_gated(_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), gate, _ptr(beta),
                                        _ptr(S), _ptr(out), N, H, dk, dv, code, _stream(dev))
    _check("kda_recurrent_step_gated", st)
    return out


def recurrent_steps(q, k, v, log_alpha, beta, S, accept=None, *, out=None, return_output=True):
    """m decode steps per sequence in one call, state updated in place
    (multi-token or speculative decoding).  q, k, v: [N, m, H, 128];
    log_alpha: [N, m, H, 128] fp32, [N, m, H] fp32 or None; beta: [N, m, H];
    S: [N, H, 128, 128] fp32; accept: None (all m tokens) or an int32 device
    tensor [N] (sequence n applies its first accept[n] tokens).  Returns o
    [N, m, H, 128] (entries of tokens not applied are left as allocated) or
    None with return_output=False."""
    import torch
    N, m, H, dk = q.shape
    dv = v.shape[-1]
    dev, dt = q.device, q.dtype
    code = _dtype_code(q)
    for t, n, shp in ((k, "k", q.shape), (v, "v", (N, m, H, dv)), (beta, "beta", (N, m, H))):
        _need(t, n, dt, shp, dev)
    gate = _gate(log_alpha, 4)
    if gate != KDA_GATE_NONE:
        _need(log_alpha, "log_alpha", torch.float32, q.shape if gate == KDA_GATE_CHANNEL else (N, m, H), dev)
    _need(S, "S", torch.float32, (N, H, dk, dv), dev)
    if accept is not None:
        _need(accept, "accept", torch.int32, (N,), dev)
    if out is None and return_output:
        out = torch.empty((N, m, H, dv), dtype=dt, device=dev)
    elif out is not None:
        _need(out, "out", dt, (N, m, H, dv), dev)
    st = lib().kda_recurrent_steps(_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), gate, _ptr(beta), _ptr(accept),
                                   _ptr(S), _ptr(out), N, m, H, dk, dv, code, _stream(dev))
    _check("kda_recurrent_steps", st)
    return out


# weight arguments of kda_layer_fwd, in call order
LAYER_WEIGHTS = ("W_q", "W_k", "W_v", "W_g", "conv_q", "conv_k", "conv_v",
                 "W_down", "W_up", "W_beta", "W_o")


def layer_workspace_layout(B, T, d_model, H, rank):
    """(total bytes, {region: byte offset}) of kda_layer_fwd's workspace."""
    offs = (ctypes.c_size_t * len(LAYER_REGIONS))()
    total = int(lib().kda_layer_workspace_layout(B, T, d_model, H, rank, offs))
    if total == 0:
        raise ValueError(f"unsupported layer shape B={B} T={T} d_model={d_model} H={H} rank={rank}")
    return total, dict(zip(LAYER_REGIONS, (int(o) for o in offs)))


def _region(ws, off, dtype, shape):
    import math
    import torch
    n = math.prod(shape) * torch.empty((), dtype=dtype).element_size()
    return ws[off:off + n].view(dtype).view(shape)


def layer_fwd(x, weights, H, *, out=None, workspace=None, intermediates=False):
    """One KDA token-mixing layer.  x: [B, T, d_model] bf16; ``weights``: dict
    with the bf16 tensors named in LAYER_WEIGHTS ([out, in]; conv taps
    [H*128, 4]).  Returns y [B, T, d_model], or (y, dict of intermediate views
    into the workspace: q, k, v, g, beta, o, zg, pre, low) with
    ``intermediates=True``."""
    import torch
    B, T, d_model = x.shape
    dev = x.device
    rank = weights["W_down"].shape[0]
    hd = H * 128
    shapes = {"W_q": (hd, d_model), "W_k": (hd, d_model), "W_v": (hd, d_model),
              "W_g": (hd, d_model), "conv_q": (hd, 4), "conv_k": (hd, 4), "conv_v": (hd, 4),
              "W_down": (rank, d_model), "W_up": (hd, rank), "W_beta": (H, d_model),
              "W_o": (d_model, hd)}
    _need(x, "x", torch.bfloat16, (B, T, d_model), dev)
    for n in LAYER_WEIGHTS:
        _need(weights[n], n, torch.bfloat16, shapes[n], dev)
    total, offs = layer_workspace_layout(B, T, d_model, H, rank)
    if out is None:
        out = torch.empty((B, T, d_model), dtype=torch.bfloat16, device=dev)
    else:
        _need(out, "out", torch.bfloat16, (B, T, d_model), dev)
    if workspace is None:
        workspace = torch.empty(total, dtype=torch.uint8, device=dev)
    if workspace.device != dev or workspace.dtype != torch.uint8 or workspace.numel() < total:
        raise ValueError(f"workspace must be a uint8 tensor of >= {total} bytes on {dev}")
    st = lib().kda_layer_fwd(_ptr(x), *(_ptr(weights[n]) for n in LAYER_WEIGHTS), _ptr(out),
                             B, T, d_model, H, rank, workspace.data_ptr(), workspace.numel(),
                             _stream(dev))
    _check("kda_layer_fwd", st)
    if not intermediates:
        return out
    ldz = (rank + H + 3) // 4 * 4
    bf, f32 = torch.bfloat16, torch.float32
    views = {
        "pre": _region(workspace, offs["pre"], bf, (B, T, 4 * hd)),
        "low": _region(workspace, offs["low"], f32, (B, T, ldz)),
        "q": _region(workspace, offs["q"], bf, (B, T, H, 128)),
        "k": _region(workspace, offs["k"], bf, (B, T, H, 128)),
        "v": _region(workspace, offs["v"], bf, (B, T, H, 128)),
        "g": _region(workspace, offs["g"], f32, (B, T, H, 128)),
        "beta": _region(workspace, offs["beta"], bf, (B, T, H)),
        "o": _region(workspace, offs["o"], bf, (B, T, H, 128)),
        "zg": _region(workspace, offs["zg"], bf, (B, T, hd)),
    }
    return out, views
