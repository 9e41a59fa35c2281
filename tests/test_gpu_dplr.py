"""GPU parity of the general diagonal-plus-low-rank forward (kda_dplr_chunk_fwd
through the C ABI) against the fp64 DPLR oracle: every output and final-state
entry at sizes the oracle finishes in seconds (several chunks, ragged tails,
both value-slice widths of the state scan), and sampled heads at the full
B = 8, H = 16, T = 4096 workload in the configuration the benchmark times."""
import numpy as np
import pytest
import torch

import gated_delta_rule_32_amd as kda
from gated_delta_rule_32_amd import inputs
from oracle import dplr_ref
from tests.kda_testutil import TOL, max_rel_err

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
NAMES = ("q", "k", "v", "a", "b", "g")


def run(inp, S0="inp", **kw):
    d = {n: (x.to(DEV) if x is not None else None) for n, x in inp.items()}
    s0 = d["S0"] if S0 == "inp" else S0
    o, S = kda.dplr_chunk_fwd(*(d[n] for n in NAMES), s0, **kw)
    torch.cuda.synchronize()
    return o, S


def check(inp, o, S, heads=None, S0="inp"):
    s0 = inp["S0"] if S0 == "inp" else S0
    args = [inp[n] for n in NAMES]
    if heads is None:
        o_ref, S_ref = dplr_ref.recurrent(*args, s0)
        eo, es = max_rel_err(o, o_ref), max_rel_err(S, S_ref)
    else:
        o_ref, S_ref = dplr_ref.recurrent(*args, s0, heads=heads)
        eo = max(max_rel_err(o[b, :, h], o_ref[i]) for i, (b, h) in enumerate(heads))
        es = max(max_rel_err(S[b, h], S_ref[i]) for i, (b, h) in enumerate(heads))
    print(f"  o err {eo:.3e}  S err {es:.3e}", flush=True)
    assert eo <= TOL["bfloat16"] and es <= TOL["bfloat16"]


@pytest.mark.parametrize("T", [1, 5, 63, 64, 65, 130, 200])
def test_ragged_lengths_with_initial_state(T):
    print(f"dplr T={T}", flush=True)
    inp = inputs.dplr_inputs(2, T, 3, g_scale=0.1, s0_std=0.05, seed=T)
    o, S = run(inp)
    check(inp, o, S)


@pytest.mark.parametrize("H", [1, 64])
def test_scan_slice_widths(H):
    """H = 1 and H = 64 select 16- and 32-column slices of the state scan."""
    print(f"dplr H={H}", flush=True)
    inp = inputs.dplr_inputs(1, 150, H, g_scale=0.05, s0_std=0.02, seed=50 + H)
    o, S = run(inp)
    check(inp, o, S, heads=[(0, 0), (0, H // 2), (0, H - 1)])


def test_no_initial_state_and_in_place_state():
    print("dplr S0=None; S_T == S0", flush=True)
    inp = inputs.dplr_inputs(1, 100, 2, g_scale=0.05, s0_std=0.05, seed=7)
    o, S = run(inp, S0=None)
    check(inp, o, S, S0=None)
    d = {n: (x.to(DEV) if x is not None else None) for n, x in inp.items()}
    state = d["S0"].clone()
    o2, S2 = kda.dplr_chunk_fwd(*(d[n] for n in NAMES), state, S_T=state)
    torch.cuda.synchronize()
    assert S2.data_ptr() == state.data_ptr()
    check(inp, o2, S2)


def test_zero_length_copies_the_state():
    inp = inputs.dplr_inputs(2, 0, 2, s0_std=0.05, seed=8)
    o, S = run(inp)
    assert o.shape == (2, 0, 2, 128)
    assert torch.equal(S.cpu(), inp["S0"])


def test_full_size_sampled_heads():
    """B = 8, H = 16, T = 4096: three sampled heads, every output and state entry."""
    print("dplr full size, sampled heads", flush=True)
    cfg = inputs.DPLR_CONFIG
    inp = inputs.dplr_inputs(cfg["B"], cfg["T"], cfg["H"], g_scale=cfg["g_scale"], s0_std=cfg["s0_std"],
                             seed=cfg["seed"])
    o, S = run(inp)
    assert torch.isfinite(o).all() and torch.isfinite(S).all()
    check(inp, o, S, heads=[(0, 0), (3, 7), (7, 15)])
