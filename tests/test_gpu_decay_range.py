"""GPU parity of the chunked prefill at strong forget gates, against the fp64
oracle.  With log-decay g = -3 softplus(N(0,1)) per token and channel the
cumulative log-decay over a 64-token chunk reaches about -150 to -250: the
chunk-start factors e^{G} and e^{-G} would leave fp32 range, so such chunks
take the sub-chunk path (reference points at the ends of the four 16-token
sub-chunks); g = -1 softplus(.) mixes chunks of both paths in one sequence.
Every schedule is covered: the fused kernel at each value-slice width and in
fp32, the two-kernel schedule, the segmented state scan, packed sequences and
the per-head gate."""
import numpy as np
import pytest
import torch

import gated_delta_rule_32_amd as kda
from gated_delta_rule_32_amd import inputs
from oracle import kda_ref
from tests.kda_testutil import TOL, max_rel_err, oracle_prefill
from tests.test_gpu_serving import channel_gate, packed

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def to_dev(inp):
    return {n: (x.to(DEV) if x is not None else None) for n, x in inp.items()}


def chunk_min_logdecay(g, T):
    """Most negative per-channel log-decay sum over any 64-token chunk (natural log)."""
    g = g.double().numpy()
    if g.ndim == 3:
        g = g[..., None]
    n = (T + 63) // 64
    pad = np.zeros((g.shape[0], n * 64 - T) + g.shape[2:])
    sums = np.concatenate([g, pad], axis=1).reshape(g.shape[0], n, 64, *g.shape[2:]).sum(axis=2)
    return float(sums.min())


def run_check(inp, workspace, tol):
    d = to_dev(inp)
    o, S = kda.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["S0"], workspace=workspace)
    torch.cuda.synchronize()
    assert torch.isfinite(o.float()).all() and torch.isfinite(S).all()
    o_ref, S_ref = oracle_prefill({**inp, "g": channel_gate(inp["g"], inp["q"])})
    eo, es = max_rel_err(o, o_ref), max_rel_err(S, S_ref)
    print(f"  o err {eo:.3e}  S err {es:.3e}  (tol {tol})", flush=True)
    assert eo <= tol and es <= tol


@pytest.mark.parametrize("dtype,B,H", [("bfloat16", 2, 64), ("bfloat16", 1, 100), ("bfloat16", 1, 3),
                                       ("float32", 1, 3)])
@pytest.mark.parametrize("g_scale", [1.0, 3.0])
def test_fused_strong_decay(dtype, B, H, g_scale):
    """Fused kernel (128 heads: 64-column slices; 100 heads: 32; 3 heads: 16 / fp32)."""
    T = 333
    print(f"strong decay fused dtype={dtype} B={B} H={H} g_scale={g_scale}", flush=True)
    inp = inputs.prefill_inputs(B, T, H, dtype=dtype, g_scale=g_scale, s0_std=0.05, seed=700 + H)
    print(f"  most negative chunk log-decay {chunk_min_logdecay(inp['g'], T):.1f}", flush=True)
    run_check(inp, None, TOL[dtype])


@pytest.mark.parametrize("B,H,T", [(1, 3, 1000), (1, 16, 1000), (1, 40, 777)])
def test_two_kernel_and_segmented_strong_decay(B, H, T):
    """Two-kernel schedule: one-pass scan (plain workspace) and, with 16
    heads or fewer and the library's workspace, the segmented scan."""
    print(f"strong decay two-kernel B={B} H={H} T={T}", flush=True)
    inp = inputs.prefill_inputs(B, T, H, dtype="bfloat16", g_scale=3.0, s0_std=0.05, seed=800 + T)
    print(f"  most negative chunk log-decay {chunk_min_logdecay(inp['g'], T):.1f}", flush=True)
    one_pass = torch.empty(kda.scan_workspace_bytes(B, T, H), dtype=torch.uint8, device=DEV)
    run_check(inp, one_pass, TOL["bfloat16"])
    nbytes = kda.workspace_size(B, T, H, kda.KDA_BF16)
    if nbytes > kda.scan_workspace_bytes(B, T, H):
        print("  segmented scan", flush=True)
        run_check(inp, torch.empty(nbytes, dtype=torch.uint8, device=DEV), TOL["bfloat16"])


def test_per_head_gate_strong_decay():
    """Gated DeltaNet gate (one decay per head and token) at g = -3 softplus(.)."""
    print("strong decay per-head gate", flush=True)
    inp = inputs.prefill_inputs(2, 300, 3, dtype="bfloat16", g_scale=3.0, s0_std=0.05, seed=901, gate="head")
    for ws in (None, torch.empty(kda.scan_workspace_bytes(2, 300, 3), dtype=torch.uint8, device=DEV)):
        run_check(inp, ws, TOL["bfloat16"])


@pytest.mark.parametrize("dtype,H", [("bfloat16", 3), ("float32", 2)])
def test_varlen_strong_decay(dtype, H):
    lengths = [65, 1, 200, 64, 130]
    print(f"strong decay varlen dtype={dtype} H={H}", flush=True)
    inp, S0, cu = packed(lengths, H, dtype, "channel", seed=31, g_scale=3.0)
    d = {n: (x[0].to(DEV) if x is not None and n != "S0" else None) for n, x in inp.items()}
    o, S = kda.chunk_fwd_varlen(d["q"], d["k"], d["v"], d["g"], d["beta"],
                                torch.from_numpy(cu).to(DEV), S0.to(DEV))
    torch.cuda.synchronize()
    for s, (a, e) in enumerate(zip(cu[:-1], cu[1:])):
        sl = lambda x: x[:, a:e]   # noqa: E731
        o_ref, S_ref = kda_ref.recurrent(sl(inp["q"]), sl(inp["k"]), sl(inp["v"]), sl(inp["g"]),
                                         sl(inp["beta"]), S0[s:s + 1])
        eo, es = max_rel_err(o[a:e], o_ref[0]), max_rel_err(S[s:s + 1], S_ref)
        print(f"  seq {s} (T={e - a}): o err {eo:.3e}  S err {es:.3e}", flush=True)
        assert eo <= TOL[dtype] and es <= TOL[dtype]
