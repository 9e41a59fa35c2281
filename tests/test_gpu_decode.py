"""GPU parity of the recurrent decode step (kda_recurrent_step through the C ABI)
against the fp64 oracle.  The oracle runs each sampled head's token stream as
one sequence: decoding step by step is the recurrence of eq. (1) over time."""
import numpy as np
import pytest
import torch

import gated_delta_rule_32_amd as kda
from gated_delta_rule_32_amd import inputs
from oracle import kda_ref
from tests.kda_testutil import TOL, max_rel_err, max_rel_err_per_head

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def run_steps(S, toks):
    outs = []
    for s in range(toks["q"].shape[0]):
        outs.append(kda.recurrent_step(toks["q"][s], toks["k"][s], toks["v"][s],
                                       toks["g"][s], toks["beta"][s], S))
    return torch.stack(outs)


def oracle_heads(S0, toks, pairs):
    """Oracle o [steps, len(pairs), 128] and final S [len(pairs), 128, 128]."""
    os_, Ss = [], []
    for n, h in pairs:
        seq = lambda x: x[:, n, h].cpu()[None, :, None]          # [1, steps, 1, .]
        o, S = kda_ref.recurrent(seq(toks["q"]), seq(toks["k"]), seq(toks["v"]),
                                 seq(toks["g"]), toks["beta"][:, n, h].cpu()[None, :, None],
                                 S0[n:n + 1, h:h + 1].cpu())
        os_.append(o[0, :, 0])
        Ss.append(S[0, 0])
    return np.stack(os_, axis=1), np.stack(Ss)


@pytest.mark.parametrize("dtype", ["float32", "bfloat16"])
def test_decode_small_all_heads(dtype):
    N, H, steps = 3, 5, 24
    print(f"decode small dtype={dtype} N={N} H={H} steps={steps}", flush=True)
    S = inputs.decode_state(N, H, s_std=0.02, seed=11, device=DEV)
    S0 = S.clone()
    toks = inputs.decode_tokens(N, H, steps, dtype=dtype, seed=11, device=DEV)
    o = run_steps(S, toks)
    torch.cuda.synchronize()
    pairs = [(n, h) for n in range(N) for h in range(H)]
    o_ref, S_ref = oracle_heads(S0, toks, pairs)
    o_gpu = o.float().cpu().numpy().reshape(steps, N * H, 128)
    tol = TOL[dtype]
    eo = max(max_rel_err(o_gpu[s], o_ref[s]) for s in range(steps))
    es = max_rel_err(S.cpu().numpy().reshape(N * H, 128, 128), S_ref)
    print(f"  worst step o err {eo:.3e}  S err {es:.3e}", flush=True)
    assert eo <= tol and es <= tol


def test_decode_full_size_all_heads():
    """256 sequences x 32 heads, 1000 steps (the decode workload): o of every
    head at steps 1, 10, 100 and 1000, and every head's final state, against
    the oracle (each head's token stream run as one sequence), globally and
    per head."""
    cfg = inputs.DECODE_CONFIG
    N, H, steps = cfg["N"], cfg["H"], cfg["steps"]
    print(f"decode full N={N} H={H} steps={steps}", flush=True)
    S = inputs.decode_state(N, H, s_std=cfg["s_std"], seed=cfg["seed"], device=DEV)
    S0 = S.cpu()
    toks = inputs.decode_tokens(N, H, steps, dtype=cfg["dtype"], seed=cfg["seed"], device=DEV)
    keep = (0, 9, 99, 999)
    o_keep = {}
    for s in range(steps):
        o = kda.recurrent_step(toks["q"][s], toks["k"][s], toks["v"][s], toks["g"][s],
                               toks["beta"][s], S)
        if s in keep:
            o_keep[s] = o.float().cpu().numpy()             # [N, H, 128]
    S_gpu = S.cpu().numpy()
    print("  gpu steps done; oracle in groups of 32 sequences", flush=True)
    worst = {s: 0.0 for s in keep}
    worst_S, worst_head = 0.0, 0.0
    o_ref_keep = {s: np.empty((N, H, 128)) for s in keep}
    S_ref = np.empty((N, H, 128, 128))
    G = 32
    for n0 in range(0, N, G):
        sl = lambda x: x[:, n0:n0 + G].transpose(0, 1).cpu()      # [G, steps, H, .]
        o_r, S_r = kda_ref.recurrent(sl(toks["q"]), sl(toks["k"]), sl(toks["v"]), sl(toks["g"]),
                                     sl(toks["beta"]), S0[n0:n0 + G])
        for s in keep:
            o_ref_keep[s][n0:n0 + G] = o_r[:, s]
        S_ref[n0:n0 + G] = S_r
    for s in keep:
        worst[s] = max_rel_err(o_keep[s], o_ref_keep[s])
        worst_head = max(worst_head, max_rel_err_per_head(o_keep[s], o_ref_keep[s], (0, 1)))
    worst_S = max_rel_err(S_gpu, S_ref)
    worst_head = max(worst_head, max_rel_err_per_head(S_gpu, S_ref, (0, 1)))
    print(f"  o err at steps 1/10/100/1000: {worst[0]:.3e} {worst[9]:.3e} {worst[99]:.3e} "
          f"{worst[999]:.3e}; S err {worst_S:.3e}; per-head worst {worst_head:.3e}", flush=True)
    tol = TOL["bfloat16"]
    assert max(worst.values()) <= tol and worst_S <= tol and worst_head <= tol


def test_decode_is_deterministic_and_zero_sized_is_noop():
    N, H = 4, 8
    S1 = inputs.decode_state(N, H, seed=3, device=DEV)
    S2 = S1.clone()
    toks = inputs.decode_tokens(N, H, 3, seed=3, device=DEV)
    o1 = run_steps(S1, toks)
    o2 = run_steps(S2, toks)
    assert torch.equal(o1, o2) and torch.equal(S1, S2)
    e = torch.empty((0, H, 128), device=DEV, dtype=torch.bfloat16)
    Se = torch.empty((0, H, 128, 128), device=DEV)
    out = kda.recurrent_step(e, e, e, e.float(), torch.empty((0, H), device=DEV,
                                                              dtype=torch.bfloat16), Se)
    assert out.shape == (0, H, 128)


def test_decode_step_continues_prefill():
    """Prefill of T-1 tokens followed by one decode step gives the oracle's
    prefill of T tokens (last output and final state)."""
    inp = inputs.prefill_inputs(2, 97, 3, dtype="bfloat16", g_scale=0.05, s0_std=0.02, seed=21)
    d = {n: (x.to(DEV) if x is not None else None) for n, x in inp.items()}
    sl = lambda x: x[:, :-1].contiguous()
    _, S = kda.chunk_fwd(sl(d["q"]), sl(d["k"]), sl(d["v"]), sl(d["g"]), sl(d["beta"]), d["S0"])
    last = lambda x: x[:, -1].contiguous()
    o_last = kda.recurrent_step(last(d["q"]), last(d["k"]), last(d["v"]), last(d["g"]),
                                last(d["beta"]), S)
    torch.cuda.synchronize()
    o_ref, S_ref = kda_ref.recurrent(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], inp["S0"])
    eo, es = max_rel_err(o_last, o_ref[:, -1]), max_rel_err(S, S_ref)
    print(f"  o err {eo:.3e}  S err {es:.3e}", flush=True)
    assert eo <= TOL["bfloat16"] and es <= TOL["bfloat16"]
