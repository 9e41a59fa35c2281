"""GPU parity of the backward pass (kda_chunk_bwd through the C ABI) against
the fp64 gradient oracle (reverse mode through the recurrence), element by
element on every gradient at sizes the oracle finishes in seconds (several
chunks, ragged tails, with and without S0 and dS_T), and on every head of the
full B = 8, H = 16, T = 4096 workload in the launch configuration the
benchmark times (per-head normwise errors)."""
import numpy as np
import pytest
import torch

import gated_delta_rule_32_amd as kda
from gated_delta_rule_32_amd import inputs
from oracle import kda_ref
from tests.kda_testutil import TOL_GRAD, max_rel_err, max_rel_err_per_head

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
NAMES = ("dq", "dk", "dv", "dg", "dbeta", "dS0")


def run_bwd(inp, gr, with_ds0=True):
    d = {n: (x.to(DEV) if x is not None else None) for n, x in {**inp, **gr}.items()}
    out = kda.chunk_bwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["S0"], d["dO"], d["dS_T"],
                        grad_S0=with_ds0)
    torch.cuda.synchronize()
    return out


def oracle_grads(inp, gr, heads=None):
    args = [inp[n] for n in ("q", "k", "v", "g", "beta", "S0")] + [gr["dO"], gr["dS_T"]]
    if heads is None:
        return kda_ref.recurrent_grad(*args)
    outs = []
    for b, h in heads:
        one = [x[b:b + 1, :, h:h + 1] for x in args[:5]]
        s0 = None if args[5] is None else args[5][b:b + 1, h:h + 1]
        dO = args[6][b:b + 1, :, h:h + 1]
        dST = None if args[7] is None else args[7][b:b + 1, h:h + 1]
        outs.append(kda_ref.recurrent_grad(*one, s0, dO, dST))
    return outs


def check(got, ref, names=NAMES):
    errs = {}
    for n, x, r in zip(names, got, ref):
        if x is None:
            continue
        errs[n] = max_rel_err(x, r)
    print("  " + "  ".join(f"{n} {e:.2e}" for n, e in errs.items()), flush=True)
    for n, e in errs.items():
        assert e <= TOL_GRAD[n], (n, e)
    return errs


@pytest.mark.parametrize("T", [1, 5, 63, 64, 65, 130, 200])
def test_ragged_lengths_with_state_and_final_gradient(T):
    print(f"backward ragged T={T}", flush=True)
    inp = inputs.prefill_inputs(2, T, 3, dtype="bfloat16", g_scale=0.1, s0_std=0.05, seed=T)
    gr = inputs.grad_inputs(2, T, 3, ds_std=0.05, seed=T)
    check(run_bwd(inp, gr), oracle_grads(inp, gr))


@pytest.mark.parametrize("T", [64, 150])
def test_no_initial_state_no_final_gradient(T):
    print(f"backward S0=None dS_T=None T={T}", flush=True)
    inp = inputs.prefill_inputs(1, T, 2, dtype="bfloat16", g_scale=0.05, seed=100 + T)
    gr = inputs.grad_inputs(1, T, 2, seed=100 + T)
    got = run_bwd(inp, gr)
    check(got, oracle_grads(inp, gr))


@pytest.mark.parametrize("B,H,T,g_scale", [(1, 3, 200, 1.0), (1, 3, 200, 3.0), (2, 64, 130, 3.0)])
def test_strong_decay(B, H, T, g_scale):
    """Per-channel log-decay g = -g_scale softplus(N(0,1)): chunk sums of the
    log-decay down to about -250 at g_scale 3 (sub-chunk references in the
    forward recomputation and in the gradient kernel); every gradient against
    the oracle, with S0 and dS_T.  128 heads select the 64-column scans."""
    print(f"backward strong decay B={B} H={H} T={T} g_scale={g_scale}", flush=True)
    inp = inputs.prefill_inputs(B, T, H, dtype="bfloat16", g_scale=g_scale, s0_std=0.05, seed=900 + H)
    gr = inputs.grad_inputs(B, T, H, ds_std=0.05, seed=900 + H)
    got = run_bwd(inp, gr)
    for x in got:
        assert torch.isfinite(x.float()).all()
    check(got, oracle_grads(inp, gr))


def test_without_ds0_output():
    print("backward without dS0", flush=True)
    inp = inputs.prefill_inputs(1, 100, 2, dtype="bfloat16", g_scale=0.05, s0_std=0.02, seed=5)
    gr = inputs.grad_inputs(1, 100, 2, ds_std=0.02, seed=5)
    got = run_bwd(inp, gr, with_ds0=False)
    assert got[5] is None
    check(got[:5], oracle_grads(inp, gr)[:5], NAMES[:5])


@pytest.mark.parametrize("H", [1, 64])
def test_scan_slice_widths(H):
    """H = 1 and H = 64 select 16- and 32-column slices in both state scans."""
    print(f"backward slice widths H={H}", flush=True)
    inp = inputs.prefill_inputs(1, 150, H, dtype="bfloat16", g_scale=0.05, s0_std=0.02, seed=H)
    gr = inputs.grad_inputs(1, 150, H, ds_std=0.02, seed=H)
    got = run_bwd(inp, gr)
    heads = [(0, 0), (0, H - 1), (0, H // 2)]
    refs = oracle_grads(inp, gr, heads)
    for (b, h), ref in zip(heads, refs):
        one = [x[b:b + 1, :, h:h + 1] for x in got[:5]] + [got[5][b:b + 1, h:h + 1]]
        check(one, ref)


def test_beta_zero_and_gate_one():
    """beta = 0 (no writes: dk = dv = 0 exactly) and g = 0 (no decay)."""
    print("backward beta=0, g=0", flush=True)
    inp = inputs.prefill_inputs(1, 130, 2, dtype="bfloat16", g_scale=0.1, s0_std=0.05, seed=9)
    inp["beta"] = torch.zeros_like(inp["beta"])
    gr = inputs.grad_inputs(1, 130, 2, ds_std=0.05, seed=9)
    got = run_bwd(inp, gr)
    assert torch.count_nonzero(got[1]) == 0 and torch.count_nonzero(got[2]) == 0
    check(got, oracle_grads(inp, gr))
    inp = inputs.prefill_inputs(1, 130, 2, dtype="bfloat16", g_scale=0.0, s0_std=0.05, seed=10)
    gr = inputs.grad_inputs(1, 130, 2, ds_std=0.05, seed=10)
    check(run_bwd(inp, gr), oracle_grads(inp, gr))


# head axes of each gradient: [B, T, H, ...] tensors and dbeta [B, T, H]
# by (batch, head); dS0 [B, H, d, d] by (batch, head)
HEAD_AXES = {"dq": (0, 2), "dk": (0, 2), "dv": (0, 2), "dg": (0, 2), "dbeta": (0, 2), "dS0": (0, 1)}


def check_per_head(got, ref):
    """Every gradient of every head: the worst per-head normwise error (each
    head judged on its own scale) within the gradient tolerance."""
    errs = {}
    for n, x, r in zip(NAMES, got, ref):
        if x is None:
            continue
        errs[n] = (max_rel_err(x, r), max_rel_err_per_head(x, r, HEAD_AXES[n]))
    print("  " + "  ".join(f"{n} {e:.2e}/{ph:.2e}" for n, (e, ph) in errs.items()), flush=True)
    for n, (_, ph) in errs.items():
        assert ph <= TOL_GRAD[n], (n, ph)


def test_config2_full_size_all_heads():
    """B = 8, H = 16, T = 4096 (the benchmarked backward workload, in the
    launch configuration the benchmark times): every gradient of all 128
    heads against the oracle."""
    print("backward c2 full size, all heads", flush=True)
    inp = inputs.prefill_config("c2_bf16_B8_H16_T4096")
    gr = inputs.grad_inputs(8, 4096, 16, seed=2)
    check_per_head(run_bwd(inp, gr), oracle_grads(inp, gr))


def gate_oracle_inputs(inp, gate, d=128):
    """The per-channel g the oracle takes for a per-head gate (the decay copied
    to every channel) or for no gate (g = 0)."""
    B, T, H, _ = inp["q"].shape
    o = dict(inp)
    if gate == "head":
        o["g"] = inp["g"][..., None].expand(B, T, H, d).contiguous()
    else:
        o["g"] = torch.zeros((B, T, H, d), dtype=torch.float32)
    return o


def reduce_gate(ref, gate):
    """Oracle gradients in the gate's own shape: dg summed over channels for a
    per-head gate (the one decay enters every channel), absent without one."""
    ref = list(ref)
    ref[3] = ref[3].sum(axis=-1) if gate == "head" else None
    return ref


@pytest.mark.parametrize("gate", ["head", "none"])
@pytest.mark.parametrize("T", [1, 65, 200])
def test_gate_variants(gate, T):
    """Gated DeltaNet (one decay per head and token) and DeltaNet (no decay)."""
    print(f"backward gate={gate} T={T}", flush=True)
    inp = inputs.prefill_inputs(2, T, 3, dtype="bfloat16", g_scale=0.1, s0_std=0.05, seed=40 + T, gate=gate)
    gr = inputs.grad_inputs(2, T, 3, ds_std=0.05, seed=40 + T)
    got = run_bwd(inp, gr)
    if gate == "head":
        assert got[3].shape == (2, T, 3)
    else:
        assert got[3] is None
    check(got, reduce_gate(oracle_grads(gate_oracle_inputs(inp, gate), gr), gate))


def test_per_head_gate_strong_decay():
    """Gated DeltaNet gate at g = -3 softplus(N(0,1)) per head and token."""
    print("backward per-head gate, strong decay", flush=True)
    inp = inputs.prefill_inputs(2, 200, 3, dtype="bfloat16", g_scale=3.0, s0_std=0.05, seed=44, gate="head")
    gr = inputs.grad_inputs(2, 200, 3, ds_std=0.05, seed=44)
    check(run_bwd(inp, gr), reduce_gate(oracle_grads(gate_oracle_inputs(inp, "head"), gr), "head"))


@pytest.mark.parametrize("name,gate", [("c2_gdn_bf16_B8_H16_T4096", "head"),
                                       ("c2_deltanet_bf16_B8_H16_T4096", "none")])
def test_gate_variants_full_size_all_heads(name, gate):
    """B = 8, H = 16, T = 4096 with the other two gates: every gradient of all
    128 heads."""
    print(f"backward {name}, all heads", flush=True)
    inp = inputs.prefill_config(name)
    gr = inputs.grad_inputs(8, 4096, 16, seed=2)
    got = run_bwd(inp, gr)
    check_per_head(got, reduce_gate(oracle_grads(gate_oracle_inputs(inp, gate), gr), gate))


def test_one_round_slices_with_ragged_tail():
    """128 heads select 64-column slices in both state scans (one round of
    workgroups); T = 150 leaves a ragged last chunk.  Every gradient of every
    head against the oracle."""
    print("backward 128 heads (64-column scan slices), T=150", flush=True)
    inp = inputs.prefill_inputs(2, 150, 64, dtype="bfloat16", g_scale=0.1, s0_std=0.05, seed=77)
    gr = inputs.grad_inputs(2, 150, 64, ds_std=0.05, seed=77)
    check(run_bwd(inp, gr), oracle_grads(inp, gr))


@pytest.mark.parametrize("B,H", [(1, 64), (3, 30)])
def test_32_column_slices_with_ragged_tail(B, H):
    """64 to 127 heads select 32-column slices (two consumer waves) in both
    state scans; T = 150 leaves a ragged last chunk, with S0, dS_T and strong
    decay.  Every gradient of every head against the oracle."""
    print(f"backward {B * H} heads (32-column scan slices), T=150", flush=True)
    inp = inputs.prefill_inputs(B, 150, H, dtype="bfloat16", g_scale=1.0, s0_std=0.05, seed=78 + H)
    gr = inputs.grad_inputs(B, 150, H, ds_std=0.05, seed=78 + H)
    check(run_bwd(inp, gr), oracle_grads(inp, gr))
