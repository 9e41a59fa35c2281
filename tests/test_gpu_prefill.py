"""GPU parity of the chunked prefill (kda_chunk_fwd through the C ABI) against
the fp64 oracle, element by element on every output and final-state entry, at
sizes the oracle finishes in seconds (several chunks, ragged tails), and on
every head at the full workload sizes in the launch configuration the
benchmark times."""
import numpy as np
import pytest
import torch

import gated_delta_rule_32_amd as kda
from gated_delta_rule_32_amd import inputs
from tests.kda_testutil import TOL, max_rel_err, max_rel_err_per_head, oracle_prefill

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def to_dev(inp):
    return {n: (x.to(DEV) if x is not None else None) for n, x in inp.items()}


def run(d, S0="inp", schedule="auto", **kw):
    """schedule: "auto" (library's choice), "fused" (no workspace) or
    "two_kernel" (a workspace large enough for the prep + scan kernels)."""
    s0 = d["S0"] if S0 == "inp" else S0
    if schedule == "fused":
        kw["workspace"] = None
    elif schedule == "two_kernel":
        B, T, H, _ = d["q"].shape
        kw["workspace"] = torch.empty(kda.scan_workspace_bytes(B, T, H), dtype=torch.uint8,
                                      device=d["q"].device)
    o, S = kda.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], s0, **kw)
    torch.cuda.synchronize()
    return o, S


def check(inp, o, S, tol, heads=None, per_head=False):
    if heads is None:
        o_ref, S_ref = oracle_prefill(inp)
        eo, es = max_rel_err(o, o_ref), max_rel_err(S, S_ref)
        if per_head:
            # each (batch, head) slice on its own scale
            ho, hs = max_rel_err_per_head(o, o_ref, (0, 2)), max_rel_err_per_head(S, S_ref, (0, 1))
            print(f"  per-head worst: o {ho:.3e}  S {hs:.3e}", flush=True)
            assert ho <= tol and hs <= tol
    else:
        refs = oracle_prefill(inp, heads)
        eo = max(max_rel_err(o[b, :, h], r[0][0, :, 0]) for (b, h), r in zip(heads, refs))
        es = max(max_rel_err(S[b, h], r[1][0, 0]) for (b, h), r in zip(heads, refs))
    print(f"  o err {eo:.3e}  S err {es:.3e}  (tol {tol})", flush=True)
    assert eo <= tol and es <= tol
    return eo, es


def test_config1_fp32_full():
    """1 head, T = 256, fp32 everywhere, S0 = 0: max relative error <= 1e-4."""
    print("prefill c1 fp32 T=256", flush=True)
    inp = inputs.prefill_config("c1_fp32_T256")
    o, S = run(to_dev(inp))
    check(inp, o, S, TOL["float32"])


@pytest.mark.parametrize("dtype,schedule", [("float32", "fused"), ("bfloat16", "fused"),
                                            ("bfloat16", "two_kernel")])
@pytest.mark.parametrize("T", [1, 5, 63, 64, 65, 130, 200])
def test_ragged_lengths_with_initial_state(dtype, schedule, T):
    print(f"prefill ragged dtype={dtype} schedule={schedule} T={T}", flush=True)
    inp = inputs.prefill_inputs(2, T, 3, dtype=dtype, g_scale=0.1, s0_std=0.05, seed=T)
    o, S = run(to_dev(inp), schedule=schedule)
    check(inp, o, S, TOL[dtype])


@pytest.mark.parametrize("B,H,T,s0_std,g_scale", [
    (1, 16, 520, 0.05, 0.1),     # 3 segments of 3 chunks (ragged last chunk)
    (1, 16, 1000, 0.0, 0.1),     # no initial state
    (1, 16, 4096, 0.05, 0.05),   # 4 segments of 16 chunks
    (2, 3, 2000, 0.05, 0.1),     # 6 heads: 8 segments of 4 chunks (ragged last chunk)
    (1, 1, 777, 0.05, 0.1),      # one head: 5 segments of 3 chunks (the last of 1.1)
    (1, 4, 1500, 0.05, 1.0),     # 12 segments of 2 chunks, strong decay
])
def test_segmented_scan(B, H, T, s0_std, g_scale):
    """16 heads or fewer with the library's workspace: the two-kernel schedule
    runs each head's state scan in segments (segment summaries, their combine,
    then every segment from its entry state).  Every output and final-state
    entry against the oracle."""
    print(f"prefill segmented scan B={B} H={H} T={T} s0_std={s0_std} g_scale={g_scale}", flush=True)
    ws = kda.workspace_size(B, T, H, kda.KDA_BF16)
    assert ws > kda.scan_workspace_bytes(B, T, H)      # room for the segment buffers
    inp = inputs.prefill_inputs(B, T, H, dtype="bfloat16", g_scale=g_scale, s0_std=s0_std, seed=300 + T)
    d = to_dev(inp)
    o, S = run(d, workspace=torch.empty(ws, dtype=torch.uint8, device=DEV))
    check(inp, o, S, TOL["bfloat16"])
    # the same call without the segment buffers (one pass per head) agrees to rounding
    o2, S2 = run(d, schedule="two_kernel")
    check(inp, o2, S2, TOL["bfloat16"])


@pytest.mark.parametrize("B,H,T,gate", [
    (1, 24, 1000, "channel"),   # 3 heads per XCD, ragged last chunk
    (2, 16, 777, "channel"),    # 32 heads
    (1, 40, 300, "channel"),
    (1, 48, 130, "channel"),    # 6 heads per XCD: 8 producers per XCD
    (3, 8, 65, "channel"),      # two chunks
    (1, 32, 500, "head"),
    (1, 32, 500, "none"),
])
def test_pipelined_schedule(B, H, T, gate):
    """24 to 48 heads (a multiple of 8) with the library's workspace: prep and
    scan in one launch, the scan waiting on per-block ready flags.  Every
    output and final-state entry against the oracle, and bitwise equal to the
    one-pass two-kernel schedule (the same products in the same order)."""
    print(f"prefill pipelined B={B} H={H} T={T} gate={gate}", flush=True)
    ws = kda.workspace_size(B, T, H, kda.KDA_BF16)
    assert ws > kda.scan_workspace_bytes(B, T, H)      # room for the flags
    inp = inputs.prefill_inputs(B, T, H, dtype="bfloat16", g_scale=0.1, s0_std=0.05, seed=400 + T, gate=gate)
    d = to_dev(inp)
    o, S = run(d, workspace=torch.empty(ws, dtype=torch.uint8, device=DEV))
    g = inp["g"] if gate == "channel" else (torch.zeros(inp["q"].shape) if inp["g"] is None
                                             else inp["g"][..., None].expand(inp["q"].shape).contiguous())
    check({**inp, "g": g}, o, S, TOL["bfloat16"])
    o2, S2 = run(d, schedule="two_kernel")
    assert torch.equal(o, o2) and torch.equal(S, S2)
    # twice more on the same workspace (flags cleared per call), S_T in place of S0
    state = d["S0"].clone()
    o3, _ = kda.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], state, S_T=state,
                          workspace=torch.empty(ws, dtype=torch.uint8, device=DEV))
    torch.cuda.synchronize()
    assert torch.equal(o3, o) and torch.equal(state, S)


def test_segmented_scan_in_place_state():
    """The segmented scan with S_T written over S0 (the same tensor)."""
    print("prefill segmented scan, S_T in place of S0", flush=True)
    B, T, H = 1, 1000, 16
    inp = inputs.prefill_inputs(B, T, H, dtype="bfloat16", g_scale=0.1, s0_std=0.05, seed=350)
    d = to_dev(inp)
    ws = torch.empty(kda.workspace_size(B, T, H, kda.KDA_BF16), dtype=torch.uint8, device=DEV)
    state = d["S0"].clone()
    o, S = kda.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], state, S_T=state, workspace=ws)
    torch.cuda.synchronize()
    assert S.data_ptr() == state.data_ptr()
    check(inp, o, state, TOL["bfloat16"])


@pytest.mark.parametrize("T", [1, 5, 63, 64, 65, 130, 200])
def test_128_heads_ragged_lengths(T):
    """128 heads select the fused kernel with 64-column value slices (two
    workgroups per head): every output and state entry, ragged tails."""
    print(f"prefill 128 heads B=2 H=64 T={T}", flush=True)
    inp = inputs.prefill_inputs(2, T, 64, dtype="bfloat16", g_scale=0.1, s0_std=0.05, seed=100 + T)
    o, S = run(to_dev(inp))
    check(inp, o, S, TOL["bfloat16"])


def test_128_heads_strong_decay():
    """Chunk sums of the log-decay down to about -65 with 64-column slices."""
    print("prefill 128 heads strong decay", flush=True)
    inp = inputs.prefill_inputs(1, 200, 128, dtype="bfloat16", g_scale=1.0, s0_std=0.05, seed=8)
    o, S = run(to_dev(inp))
    check(inp, o, S, TOL["bfloat16"])


@pytest.mark.parametrize("schedule", ["fused", "two_kernel"])
@pytest.mark.parametrize("H", [1, 40, 100, 128])
def test_bf16_slice_widths(H, schedule):
    """Head counts that select each value-slice width (16, 32, 64 columns)."""
    print(f"prefill slice widths H={H} schedule={schedule}", flush=True)
    inp = inputs.prefill_inputs(1, 150, H, dtype="bfloat16", g_scale=0.05, s0_std=0.02, seed=H)
    o, S = run(to_dev(inp), schedule=schedule)
    heads = [(0, 0), (0, H - 1), (0, H // 2)]
    check(inp, o, S, TOL["bfloat16"], heads=heads)


@pytest.mark.parametrize("schedule", ["fused", "two_kernel"])
def test_config2_reduced_all_elements(schedule):
    print(f"prefill c2 reduced B=2 H=4 T=1000 schedule={schedule}", flush=True)
    inp = inputs.prefill_config("c2_bf16_B8_H16_T4096", B=2, H=4, T=1000)
    o, S = run(to_dev(inp), schedule=schedule)
    check(inp, o, S, TOL["bfloat16"])


@pytest.mark.parametrize("schedule", ["auto", "two_kernel"])
def test_config2_full_size_all_heads(schedule):
    """B = 8, H = 16, T = 4096 bf16: every output and state entry of all 128
    heads, globally and per head."""
    print(f"prefill c2 full schedule={schedule}", flush=True)
    inp = inputs.prefill_config("c2_bf16_B8_H16_T4096")
    o, S = run(to_dev(inp), schedule=schedule)
    check(inp, o, S, TOL["bfloat16"], per_head=True)


@pytest.mark.parametrize("schedule", ["auto", "fused"])
def test_config3_full_size_all_heads(schedule):
    """B = 1, H = 32, T = 65536 bf16, S0 ~ N(0, 0.02^2): every output and
    state entry of all 32 heads (1024 chunks each), globally and per head."""
    print(f"prefill c3 full schedule={schedule}", flush=True)
    inp = inputs.prefill_config("c3_bf16_B1_H32_T65536")
    o, S = run(to_dev(inp), schedule=schedule)
    o = o.cpu()
    torch.cuda.empty_cache()
    check(inp, o, S, TOL["bfloat16"], per_head=True)


def test_strong_decay_near_range_limit():
    """Per-channel log-decay of about -0.8 per token: chunk sums down to about -65."""
    print("prefill strong decay", flush=True)
    inp = inputs.prefill_inputs(1, 200, 2, dtype="bfloat16", g_scale=1.0, s0_std=0.05, seed=8)
    for schedule in ("fused", "two_kernel"):
        o, S = run(to_dev(inp), schedule=schedule)
        check(inp, o, S, TOL["bfloat16"])
    inp32 = inputs.prefill_inputs(1, 200, 2, dtype="float32", g_scale=1.0, s0_std=0.05, seed=8)
    o, S = run(to_dev(inp32))
    check(inp32, o, S, TOL["float32"])


def test_schedules_agree_closely():
    """Fused and two-kernel schedules compute the same products in the same
    precision; they agree far more tightly than either does with the oracle."""
    inp = inputs.prefill_inputs(2, 300, 3, dtype="bfloat16", g_scale=0.05, s0_std=0.02, seed=31)
    d = to_dev(inp)
    o1, S1 = run(d, schedule="fused")
    o2, S2 = run(d, schedule="two_kernel")
    assert max_rel_err(o2, o1.float().cpu().numpy()) <= 1e-2
    assert max_rel_err(S2, S1.cpu().numpy()) <= 1e-2


@pytest.mark.parametrize("schedule", ["fused", "two_kernel", "fused_128_heads"])
def test_state_options_and_edge_cases(schedule):
    # (128 heads without a workspace select 64-column slices)
    H = 64 if schedule == "fused_128_heads" else 2
    schedule = "fused" if schedule == "fused_128_heads" else schedule
    inp = inputs.prefill_inputs(2, 77, H, dtype="bfloat16", g_scale=0.1, s0_std=0.05, seed=5)
    d = to_dev(inp)
    go = lambda S0="inp", **kw: run(d, S0=S0, schedule=schedule, **kw)  # noqa: E731
    o_ref, S_ref = go()
    # S_T not requested
    o2, S2 = go(return_state=False)
    assert S2 is None and torch.equal(o2, o_ref)
    # in place: S_T == S0
    S_io = d["S0"].clone()
    o3, _ = go(S0=S_io, S_T=S_io)
    assert torch.equal(o3, o_ref) and torch.equal(S_io, S_ref)
    # S0 = None equals an explicit zero state
    oz, Sz = go(S0=None)
    oz2, Sz2 = go(S0=torch.zeros_like(d["S0"]))
    assert torch.equal(oz, oz2) and torch.equal(Sz, Sz2)
    # T = 0 copies the initial state (or zeros)
    e = lambda x: x[:, :0].contiguous()  # noqa: E731
    _, S0c = kda.chunk_fwd(e(d["q"]), e(d["k"]), e(d["v"]), e(d["g"]), e(d["beta"]), d["S0"])
    _, Sze = kda.chunk_fwd(e(d["q"]), e(d["k"]), e(d["v"]), e(d["g"]), e(d["beta"]), None)
    torch.cuda.synchronize()
    assert torch.equal(S0c, d["S0"]) and torch.count_nonzero(Sze) == 0
    # deterministic: bitwise equal reruns
    o4, S4 = go()
    assert torch.equal(o4, o_ref) and torch.equal(S4, S_ref)


def test_split_and_resume_matches_single_call():
    inp = inputs.prefill_inputs(1, 300, 4, dtype="bfloat16", g_scale=0.05, s0_std=0.02, seed=6)
    d = to_dev(inp)
    o, S = run(d)
    a = {n: (x[:, :128].contiguous() if x is not None and x.dim() >= 3 else x) for n, x in d.items()}
    bb = {n: (x[:, 128:].contiguous() if x is not None and x.dim() >= 3 else x) for n, x in d.items()}
    a["S0"] = d["S0"]
    oa, Sa = run(a)
    bb["S0"] = Sa
    ob, Sb = run(bb)
    o_ref, S_ref = oracle_prefill(inp)
    eo, es = max_rel_err(torch.cat([oa, ob], 1), o_ref), max_rel_err(Sb, S_ref)
    print(f"  o err {eo:.3e}  S err {es:.3e}", flush=True)
    assert eo <= TOL["bfloat16"] and es <= TOL["bfloat16"]


def test_nan_propagates():
    """NaN inputs are not masked: a NaN value in chunk 1 reaches the outputs of
    that chunk onward and the final state; chunk 0 stays finite."""
    inp = inputs.prefill_inputs(1, 150, 1, dtype="float32", seed=9)
    inp["v"][0, 70, 0, 5] = float("nan")
    o, S = run(to_dev(inp))
    assert torch.isnan(o[0, 70:]).any() and torch.isnan(S).any()
    assert not torch.isnan(o[0, :64]).any()
