"""The allocation-free prefill entry point (kda_chunk_fwd_noalloc, scratch in a
static device array of the library) against kda_chunk_fwd_gated with a
caller-supplied workspace: two calls in a row through the C ABI, the second on
a smaller input (the array keeps the first call's contents), each compared
with the workspace entry point's output and final state."""
import pytest
import torch

import gated_delta_rule_32_amd as kda
from gated_delta_rule_32_amd import inputs
from tests.kda_testutil import TOL, max_rel_err

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _stream():
    return torch.cuda.current_stream(DEV).cuda_stream


def _call_pair(B, T, H, seed):
    inp = inputs.prefill_inputs(B, T, H, dtype="bfloat16", g_scale=0.1, s0_std=0.05, seed=seed)
    d = {n: (x.to(DEV) if x is not None else None) for n, x in inp.items()}
    lib = kda.lib()
    p = lambda t: None if t is None else t.data_ptr()   # noqa: E731
    args = (p(d["q"]), p(d["k"]), p(d["v"]), p(d["g"]), kda.KDA_GATE_CHANNEL, p(d["beta"]), p(d["S0"]))
    # the existing entry point, with the workspace the library asks for
    nbytes = kda.workspace_size(B, T, H, kda.KDA_BF16)
    assert nbytes > 0, "shape must select the two-kernel schedule (scratch in use)"
    assert nbytes <= kda.lib().kda_chunk_fwd_scan_workspace_size(B, T, H, 128, 128, kda.KDA_BF16) * 4
    ws = torch.empty(nbytes, dtype=torch.uint8, device=DEV)
    o_ref = torch.empty_like(d["v"])
    S_ref = torch.empty((B, H, 128, 128), dtype=torch.float32, device=DEV)
    st = lib.kda_chunk_fwd_gated(*args, p(o_ref), p(S_ref), B, T, H, 128, 128, kda.KDA_BF16,
                                 p(ws), nbytes, _stream())
    assert st == 0, kda.status_string(st)
    # the allocation-free entry point
    o = torch.full_like(d["v"], float("nan"))
    S = torch.full((B, H, 128, 128), float("nan"), dtype=torch.float32, device=DEV)
    st = lib.kda_chunk_fwd_noalloc(*args, p(o), p(S), B, T, H, 128, 128, kda.KDA_BF16, _stream())
    assert st == 0, kda.status_string(st)
    torch.cuda.synchronize()
    eo = max_rel_err(o, o_ref.float().cpu().numpy())
    es = max_rel_err(S, S_ref.cpu().numpy())
    same = torch.equal(o, o_ref) and torch.equal(S, S_ref)
    print(f"  noalloc B={B} T={T} H={H}: o {eo:.2e} S {es:.2e} bitwise equal {same}", flush=True)
    assert eo <= TOL["bfloat16"] and es <= TOL["bfloat16"]
    assert torch.isfinite(o.float()).all() and torch.isfinite(S).all()


def test_noalloc_matches_workspace_entry_point_twice():
    print("noalloc: 16 heads x 1000 tokens (segmented scan), then 4 heads x 300 tokens", flush=True)
    _call_pair(1, 1000, 16, seed=501)
    _call_pair(1, 300, 4, seed=502)


def test_noalloc_rejects_oversized_and_runs_fused_shapes():
    lib = kda.lib()
    # 32 heads x 65536 tokens needs 2.4 GB of operand blocks: rejected on the host
    st = lib.kda_chunk_fwd_noalloc(1, 2, 3, 4, 0, 5, None, 6, 7, 1, 65536, 32, 128, 128, kda.KDA_BF16, None)
    assert st == -5
    # 128 heads: the fused kernel, no scratch; equals kda_chunk_fwd without workspace
    inp = inputs.prefill_inputs(2, 100, 64, dtype="bfloat16", g_scale=0.1, s0_std=0.05, seed=503)
    d = {n: (x.to(DEV) if x is not None else None) for n, x in inp.items()}
    o_ref, S_ref = kda.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["S0"], workspace=None)
    o = torch.empty_like(o_ref)
    S = torch.empty_like(S_ref)
    p = lambda t: t.data_ptr()   # noqa: E731
    st = lib.kda_chunk_fwd_noalloc(p(d["q"]), p(d["k"]), p(d["v"]), p(d["g"]), kda.KDA_GATE_CHANNEL,
                                   p(d["beta"]), p(d["S0"]), p(o), p(S), 2, 100, 64, 128, 128, kda.KDA_BF16,
                                   _stream())
    assert st == 0
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref) and torch.equal(S, S_ref)
