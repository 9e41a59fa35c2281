"""GPU checks of the serving path through the C ABI: variable-length packed
prefill (kda_chunk_fwd_varlen) against the fp64 oracle run on every sequence
separately; prefill -> decode hand-off of the per-sequence states; multi-token
decode steps (a few tokens through the prefill path, state updated in place);
and a decode step captured in a HIP graph, replayed several times with eager
work in between, each replay checked against the eager call."""
import numpy as np
import pytest
import torch

import gated_delta_rule_32_amd as kda
from gated_delta_rule_32_amd import inputs
from oracle import kda_ref
from tests.kda_testutil import TOL, max_rel_err

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def channel_gate(g, like):
    if g is None:
        return torch.zeros(like.shape, dtype=torch.float32)
    return g if g.shape == like.shape else g[..., None].expand(like.shape).contiguous()


def packed(lengths, H, dtype, gate, seed, g_scale=0.1):
    """Sequences of the given lengths packed along one token axis."""
    total = int(sum(lengths))
    inp = inputs.prefill_inputs(1, total, H, dtype=dtype, g_scale=g_scale, s0_std=0.0, seed=seed, gate=gate)
    S0 = torch.from_numpy(0.05 * np.random.default_rng([seed, 2]).standard_normal(
        (len(lengths), H, 128, 128), dtype=np.float32))
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    return inp, S0, cu


@pytest.mark.parametrize("gate", ["channel", "head", "none"])
@pytest.mark.parametrize("dtype,H", [("float32", 3), ("bfloat16", 3), ("bfloat16", 16)])
def test_varlen_prefill_matches_each_sequence(gate, dtype, H):
    """(8 sequences x 16 heads select 64-column slices.)"""
    lengths = [1, 63, 64, 65, 0, 130, 200, 7]
    print(f"varlen prefill gate={gate} dtype={dtype} H={H} lengths={lengths}", flush=True)
    inp, S0, cu = packed(lengths, H, dtype, gate, seed=21)
    d = {n: (x[0].to(DEV) if x is not None and n != "S0" else None) for n, x in inp.items()}
    o, S = kda.chunk_fwd_varlen(d["q"], d["k"], d["v"], d["g"], d["beta"],
                                torch.from_numpy(cu).to(DEV), S0.to(DEV))
    torch.cuda.synchronize()
    for s, (a, e) in enumerate(zip(cu[:-1], cu[1:])):
        sl = lambda x: x[:, a:e]
        o_ref, S_ref = kda_ref.recurrent(sl(inp["q"]), sl(inp["k"]), sl(inp["v"]),
                                         sl(channel_gate(inp["g"], inp["q"])), sl(inp["beta"]),
                                         S0[s:s + 1])
        es = max_rel_err(S[s:s + 1], S_ref)
        eo = max_rel_err(o[a:e], o_ref[0]) if e > a else 0.0
        print(f"  seq {s} (T={e - a}): o err {eo:.3e}  S err {es:.3e}", flush=True)
        assert eo <= TOL[dtype] and es <= TOL[dtype]


def test_varlen_prefill_then_decode_handoff():
    """Per-sequence final states of a packed prefill continue as decode states."""
    lengths, H = [70, 5, 129], 4
    inp, S0, cu = packed(lengths, H, "bfloat16", "channel", seed=22)
    d = {n: (x[0].to(DEV) if x is not None and n != "S0" else None) for n, x in inp.items()}
    _, S = kda.chunk_fwd_varlen(d["q"], d["k"], d["v"], d["g"], d["beta"],
                                torch.from_numpy(cu).to(DEV), S0.to(DEV))
    S_ref = []
    for s, (a, e) in enumerate(zip(cu[:-1], cu[1:])):
        sl = lambda x: x[:, a:e]
        S_ref.append(kda_ref.recurrent(sl(inp["q"]), sl(inp["k"]), sl(inp["v"]), sl(inp["g"]),
                                       sl(inp["beta"]), S0[s:s + 1])[1])
    S_ref = np.concatenate(S_ref)
    toks = inputs.decode_tokens(len(lengths), H, 2, seed=22, device=DEV)
    for st in range(2):
        o = kda.recurrent_step(toks["q"][st], toks["k"][st], toks["v"][st], toks["g"][st],
                               toks["beta"][st], S)
        torch.cuda.synchronize()
        seq = lambda x: x[st].cpu()[:, None]
        o_ref, S_ref = kda_ref.recurrent(seq(toks["q"]), seq(toks["k"]), seq(toks["v"]), seq(toks["g"]),
                                         toks["beta"][st].cpu()[:, None], S_ref)
        eo, es = max_rel_err(o, o_ref[:, 0]), max_rel_err(S, S_ref)
        print(f"  decode step {st}: o err {eo:.3e}  S err {es:.3e}", flush=True)
        assert eo <= TOL["bfloat16"] and es <= TOL["bfloat16"]


@pytest.mark.parametrize("m", [2, 4])
def test_multi_token_decode_in_place(m):
    """m tokens per sequence per step through the chunked path, state updated
    in place (S_T is S0), for three steps."""
    N, H = 6, 8
    S = inputs.decode_state(N, H, s_std=0.02, seed=23, device=DEV)
    S_ref = S.double().cpu().numpy()
    for st in range(3):
        inp = inputs.prefill_inputs(N, m, H, dtype="bfloat16", g_scale=0.05, seed=100 * m + st)
        d = {n: (x.to(DEV) if x is not None else None) for n, x in inp.items()}
        o, _ = kda.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], S, S_T=S, workspace=None)
        torch.cuda.synchronize()
        o_ref, S_ref = kda_ref.recurrent(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], S_ref)
        eo, es = max_rel_err(o, o_ref), max_rel_err(S, S_ref)
        print(f"  m={m} step {st}: o err {eo:.3e}  S err {es:.3e}", flush=True)
        assert eo <= TOL["bfloat16"] and es <= TOL["bfloat16"]


def test_graph_captured_decode_step_replays():
    """One decode step captured in a HIP graph (through torch.cuda.graph, on
    static buffers), replayed three times with new tokens copied in eagerly
    between replays; every replay equals the eager call bit for bit."""
    N, H, steps = 8, 32, 3
    S_graph = inputs.decode_state(N, H, s_std=0.02, seed=24, device=DEV)
    S_eager = S_graph.clone()
    toks = inputs.decode_tokens(N, H, steps, seed=24, device=DEV)
    static = {n: torch.empty_like(toks[n][0]) for n in ("q", "k", "v", "g", "beta")}
    out_static = torch.empty((N, H, 128), dtype=torch.bfloat16, device=DEV)
    # warm-up outside the graph on a scratch state
    scratch = S_graph.clone()
    for n in static:
        static[n].copy_(toks[n][0])
    kda.recurrent_step(static["q"], static["k"], static["v"], static["g"], static["beta"], scratch,
                       out=out_static)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        kda.recurrent_step(static["q"], static["k"], static["v"], static["g"], static["beta"], S_graph,
                           out=out_static)
    torch.cuda.synchronize()
    for st in range(steps):
        for n in static:
            static[n].copy_(toks[n][st])
        graph.replay()
        o_e = kda.recurrent_step(toks["q"][st], toks["k"][st], toks["v"][st], toks["g"][st],
                                 toks["beta"][st], S_eager)
        torch.cuda.synchronize()
        print(f"  replay {st}: o equal {torch.equal(out_static, o_e)}  S equal {torch.equal(S_graph, S_eager)}",
              flush=True)
        assert torch.equal(out_static, o_e) and torch.equal(S_graph, S_eager)


def test_auto_workspace_is_per_stream():
    """Two streams, each running the two-kernel schedule with the "auto"
    workspace at the same time, give exactly the results of running the two
    calls one after the other (the cached workspace is per stream)."""
    print("auto workspace on two streams", flush=True)
    d = [{n: (x.to(DEV) if x is not None else None) for n, x in
          inputs.prefill_inputs(1, 700, 4, dtype="bfloat16", seed=s).items()} for s in (31, 32)]
    args = lambda x: (x["q"], x["k"], x["v"], x["g"], x["beta"], x["S0"])
    ref = [kda.chunk_fwd(*args(x)) for x in d]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    got = []
    for x, st in zip(d, streams):
        with torch.cuda.stream(st):
            got.append(kda.chunk_fwd(*args(x)))
    torch.cuda.synchronize()
    for (o, S), (ro, rS) in zip(got, ref):
        assert torch.equal(o, ro) and torch.equal(S, rS)


@pytest.mark.parametrize("gate", ["channel", "head", "none"])
@pytest.mark.parametrize("dtype,m", [("float32", 3), ("bfloat16", 1), ("bfloat16", 8)])
def test_recurrent_steps_all_tokens(gate, dtype, m):
    """kda_recurrent_steps with every one of the m tokens applied: outputs of
    all tokens and the final state against the oracle run over the m tokens."""
    N, H = 5, 6
    print(f"recurrent_steps gate={gate} dtype={dtype} m={m}", flush=True)
    inp = inputs.prefill_inputs(N, m, H, dtype=dtype, g_scale=0.1, s0_std=0.03, seed=60 + m, gate=gate)
    d = {n: (x.to(DEV) if x is not None else None) for n, x in inp.items()}
    S = d["S0"].clone()
    o = kda.recurrent_steps(d["q"], d["k"], d["v"], d["g"], d["beta"], S)
    torch.cuda.synchronize()
    o_ref, S_ref = kda_ref.recurrent(inp["q"], inp["k"], inp["v"], channel_gate(inp["g"], inp["q"]), inp["beta"],
                                     inp["S0"])
    eo, es = max_rel_err(o, o_ref), max_rel_err(S, S_ref)
    print(f"  o err {eo:.3e}  S err {es:.3e}", flush=True)
    assert eo <= TOL[dtype] and es <= TOL[dtype]


def test_speculative_decode_accepted_prefix():
    """Speculative decoding, three rounds: m = 4 drafted tokens per sequence
    are verified from the outputs of kda_chunk_fwd run on them without
    committing the state (S_T = NULL); then kda_recurrent_steps advances each
    sequence's state by its accepted prefix accept[n] (0 .. 4) in one call.
    Against the oracle run over the accepted tokens of every round in turn;
    outputs of tokens past the prefix are left untouched."""
    N, H, m = 6, 4, 4
    S = inputs.decode_state(N, H, s_std=0.02, seed=71, device=DEV)
    S_ref = S.double().cpu().numpy()
    rng = np.random.default_rng(72)
    for rnd in range(3):
        inp = inputs.prefill_inputs(N, m, H, dtype="bfloat16", g_scale=0.1, seed=700 + rnd)
        d = {n: (x.to(DEV) if x is not None else None) for n, x in inp.items()}
        # verification pass over all drafted tokens: outputs only
        o_ver, none = kda.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], S, return_state=False,
                                    workspace=None)
        assert none is None
        o_all_ref, _ = kda_ref.recurrent(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], S_ref)
        torch.cuda.synchronize()
        assert max_rel_err(o_ver, o_all_ref) <= TOL["bfloat16"]
        accept = np.array([0, 1, 2, 3, 4] + [int(rng.integers(0, m + 1))], dtype=np.int32)[:N]
        out = torch.full_like(d["v"], float("nan"))
        kda.recurrent_steps(d["q"], d["k"], d["v"], d["g"], d["beta"], S, torch.from_numpy(accept).to(DEV),
                            out=out)
        torch.cuda.synchronize()
        for n in range(N):
            j = int(accept[n])
            sl = lambda x: x[n:n + 1, :j]   # noqa: E731
            if j > 0:
                o_r, S_n = kda_ref.recurrent(sl(inp["q"]), sl(inp["k"]), sl(inp["v"]), sl(inp["g"]),
                                             sl(inp["beta"]), S_ref[n:n + 1])
                assert max_rel_err(out[n:n + 1, :j], o_r) <= TOL["bfloat16"]
                S_ref[n] = S_n[0]
            assert torch.isnan(out[n, j:].float()).all()
        es = max_rel_err(S, S_ref)
        print(f"  round {rnd}: accept {accept.tolist()}  S err {es:.3e}", flush=True)
        assert es <= TOL["bfloat16"]
