"""GPU parity of the gate variants (kda_chunk_fwd_gated / kda_recurrent_step_gated
through the C ABI): one decay per head and token (Gated DeltaNet) and no decay
(DeltaNet), against the fp64 oracle on the same recurrence with the head's
decay on every channel (or none).  The oracle's reductions to Gated DeltaNet
and DeltaNet are pinned on the CPU."""
import pytest
import torch

import gated_delta_rule_32_amd as kda
from gated_delta_rule_32_amd import inputs
from oracle import kda_ref
from tests.kda_testutil import TOL, max_rel_err

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def channel_gate(g, like):
    """The per-channel log-decay that a per-head gate (or none) stands for."""
    if g is None:
        return torch.zeros(like.shape, dtype=torch.float32)
    return g[..., None].expand(like.shape).contiguous()


def oracle(inp):
    return kda_ref.recurrent(inp["q"], inp["k"], inp["v"], channel_gate(inp["g"], inp["q"]),
                             inp["beta"], inp["S0"])


def run(inp, schedule):
    d = {n: (x.to(DEV) if x is not None else None) for n, x in inp.items()}
    B, T, H, _ = inp["q"].shape
    ws = None
    if schedule == "two_kernel":
        ws = torch.empty(kda.scan_workspace_bytes(B, T, H), dtype=torch.uint8, device=DEV)
    o, S = kda.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["S0"], workspace=ws)
    torch.cuda.synchronize()
    return o, S


@pytest.mark.parametrize("gate", ["head", "none"])
@pytest.mark.parametrize("dtype,schedule", [("float32", "fused"), ("bfloat16", "fused"),
                                            ("bfloat16", "two_kernel")])
@pytest.mark.parametrize("T", [1, 63, 64, 65, 200])
def test_prefill_gate_variants(gate, dtype, schedule, T):
    print(f"gated prefill gate={gate} dtype={dtype} schedule={schedule} T={T}", flush=True)
    inp = inputs.prefill_inputs(2, T, 3, dtype=dtype, g_scale=0.1, s0_std=0.05, seed=T, gate=gate)
    o, S = run(inp, schedule)
    o_ref, S_ref = oracle(inp)
    eo, es = max_rel_err(o, o_ref), max_rel_err(S, S_ref)
    print(f"  o err {eo:.3e}  S err {es:.3e}", flush=True)
    assert eo <= TOL[dtype] and es <= TOL[dtype]


@pytest.mark.parametrize("gate", ["head", "none"])
def test_segmented_scan_gate_variants(gate):
    """8 heads, 1300 tokens with the library's workspace: the state scan runs
    in 7 segments of 3 chunks; every output and state entry."""
    print(f"gated prefill segmented scan gate={gate}", flush=True)
    B, T, H = 1, 1300, 8
    inp = inputs.prefill_inputs(B, T, H, dtype="bfloat16", g_scale=0.1, s0_std=0.05, seed=400, gate=gate)
    d = {n: (x.to(DEV) if x is not None else None) for n, x in inp.items()}
    ws = torch.empty(kda.workspace_size(B, T, H, kda.KDA_BF16), dtype=torch.uint8, device=DEV)
    o, S = kda.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["S0"], workspace=ws)
    torch.cuda.synchronize()
    o_ref, S_ref = oracle(inp)
    eo, es = max_rel_err(o, o_ref), max_rel_err(S, S_ref)
    print(f"  o err {eo:.3e}  S err {es:.3e}", flush=True)
    assert eo <= TOL["bfloat16"] and es <= TOL["bfloat16"]


@pytest.mark.parametrize("gate", ["head", "none"])
@pytest.mark.parametrize("T", [1, 65, 200])
def test_128_heads_gate_variants(gate, T):
    """64-column slices (128 heads) with each gate layout: every output and state entry."""
    print(f"gated prefill 128 heads gate={gate} T={T}", flush=True)
    inp = inputs.prefill_inputs(2, T, 64, dtype="bfloat16", g_scale=0.1, s0_std=0.05, seed=200 + T, gate=gate)
    o, S = run(inp, "fused")
    o_ref, S_ref = oracle(inp)
    eo, es = max_rel_err(o, o_ref), max_rel_err(S, S_ref)
    print(f"  o err {eo:.3e}  S err {es:.3e}", flush=True)
    assert eo <= TOL["bfloat16"] and es <= TOL["bfloat16"]


@pytest.mark.parametrize("gate", ["head", "none"])
@pytest.mark.parametrize("H", [40, 100, 128])
def test_prefill_gate_slice_widths(gate, H):
    """Head counts that select the 16-, 32- and 64-column fused kernels."""
    print(f"gated prefill gate={gate} H={H}", flush=True)
    inp = inputs.prefill_inputs(1, 150, H, dtype="bfloat16", g_scale=0.05, s0_std=0.02, seed=H, gate=gate)
    o, S = run(inp, "fused")
    for h in (0, H // 2, H - 1):
        one = {n: (None if x is None else (x[:, :, h:h + 1] if n != "S0" else x[:, h:h + 1]))
               for n, x in inp.items()}
        o_ref, S_ref = oracle(one)
        eo, es = max_rel_err(o[:, :, h:h + 1], o_ref), max_rel_err(S[:, h:h + 1], S_ref)
        print(f"  head {h}: o err {eo:.3e}  S err {es:.3e}", flush=True)
        assert eo <= TOL["bfloat16"] and es <= TOL["bfloat16"]


def test_head_gate_equals_broadcast_channel_gate():
    """The per-head path and the per-channel path fed the broadcast decay
    compute the same recurrence (bf16, to the kernels' rounding)."""
    inp = inputs.prefill_inputs(2, 130, 3, dtype="bfloat16", g_scale=0.1, s0_std=0.05, seed=7, gate="head")
    o_h, S_h = run(inp, "fused")
    inp_c = dict(inp, g=channel_gate(inp["g"], inp["q"]))
    o_c, S_c = run(inp_c, "fused")
    assert max_rel_err(o_h, o_c.double().cpu().numpy()) <= 2e-3
    assert max_rel_err(S_h, S_c.double().cpu().numpy()) <= 2e-3


@pytest.mark.parametrize("gate", ["head", "none"])
@pytest.mark.parametrize("dtype", ["float32", "bfloat16"])
def test_decode_gate_variants(gate, dtype):
    print(f"gated decode gate={gate} dtype={dtype}", flush=True)
    N, H, steps = 4, 8, 3
    S = inputs.decode_state(N, H, s_std=0.02, seed=11, device=DEV)
    S_ref = S.double().cpu().numpy()
    toks = inputs.decode_tokens(N, H, steps, dtype=dtype, seed=11, device=DEV, gate=gate)
    for s in range(steps):
        o = kda.recurrent_step(toks["q"][s], toks["k"][s], toks["v"][s],
                               None if toks["g"] is None else toks["g"][s], toks["beta"][s], S)
        torch.cuda.synchronize()
        seq = lambda x: x[s].cpu()[:, None]
        g = channel_gate(None if toks["g"] is None else toks["g"][s].cpu(), toks["q"][s].cpu())[:, None]
        o_ref, S_ref = kda_ref.recurrent(seq(toks["q"]), seq(toks["k"]), seq(toks["v"]), g,
                                         toks["beta"][s].cpu()[:, None], S_ref)
        eo, es = max_rel_err(o, o_ref[:, 0]), max_rel_err(S, S_ref)
        print(f"  step {s}: o err {eo:.3e}  S err {es:.3e}", flush=True)
        assert eo <= TOL[dtype] and es <= TOL[dtype]
