"""C ABI checks that need no GPU: the library loads, exports every symbol that
include/kda.h declares, and its host-side validation rejects bad arguments
before touching any memory (fake pointers are never dereferenced)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kda.h")

kda = pytest.importorskip("gated_delta_rule_32_amd")
from gated_delta_rule_32_amd import _binding  # noqa: E402

F32, BF16 = 0, 1
OK, INVALID, UNSUP, ALIGN, WSERR = 0, -1, -2, -3, -5
P = 0x10000000  # fake, 16-byte aligned "device" addresses; never dereferenced


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kda_[a-z_0-9]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_binding.LIB_PATH):
        pytest.skip("libkda.so not built")
    return _binding.lib()


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert set(names) == {"kda_chunk_fwd", "kda_chunk_fwd_workspace_size", "kda_chunk_fwd_scan_workspace_size",
                          "kda_chunk_fwd_noalloc", "kda_recurrent_steps",
                          "kda_chunk_fwd_block_bytes", "kda_chunk_bwd", "kda_chunk_bwd_gated",
                          "kda_chunk_bwd_workspace_size", "kda_chunk_fwd_gated", "kda_chunk_fwd_varlen",
                          "kda_mqa_decode", "kda_mqa_decode_workspace_size",
                          "kda_dplr_chunk_fwd", "kda_dplr_chunk_fwd_workspace_size",
                          "kda_recurrent_step_gated", "kda_recurrent_step",
                          "kda_layer_fwd", "kda_layer_workspace_layout",
                          "kda_status_string", "kda_version"}
    for n in names:
        assert hasattr(lib, n), n
    assert set(_binding.SIGNATURES) == set(names)


def test_status_strings(lib):
    for code in (OK, INVALID, UNSUP, ALIGN, -4, WSERR, 12345):
        assert isinstance(lib.kda_status_string(code), bytes)
    assert lib.kda_version().decode().count(".") == 2


def chunk(lib, q=P, k=P + 2**24, v=P + 2**25, g=P + 2**26, beta=P + 2**27, S0=None,
          o=P + 2**28, ST=P + 2**29, B=1, T=64, H=1, dk=128, dv=128, dt=BF16, ws=None, wsb=0):
    return lib.kda_chunk_fwd(q, k, v, g, beta, S0, o, ST, B, T, H, dk, dv, dt, ws, wsb, None)


def step(lib, q=P, k=P + 2**24, v=P + 2**25, g=P + 2**26, beta=P + 2**27, S=P + 2**28,
         o=P + 2**29, N=1, H=1, dk=128, dv=128, dt=BF16):
    return lib.kda_recurrent_step(q, k, v, g, beta, S, o, N, H, dk, dv, dt, None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), INVALID), (dict(k=None), INVALID), (dict(v=None), INVALID),
    (dict(g=None), INVALID), (dict(beta=None), INVALID), (dict(o=None), INVALID),
    (dict(B=-1), INVALID), (dict(T=-1), INVALID), (dict(H=-2), INVALID),
    (dict(dk=64), UNSUP), (dict(dv=256), UNSUP), (dict(dt=7), UNSUP),
    (dict(q=P + 2), ALIGN), (dict(g=P + 4), ALIGN), (dict(o=P + 2**28 + 8), ALIGN),
    (dict(S0=P + 2**30 + 4), ALIGN), (dict(beta=P + 2**27 + 1), ALIGN),
    (dict(o=P), INVALID),                       # o overlaps q
    (dict(ST=P + 2**26 + 64), INVALID),         # S_T overlaps g
    (dict(S0=P + 2**30, ST=P + 2**30 + 16), INVALID),  # partial S0/S_T overlap
    (dict(B=2**30, H=2**30), UNSUP),            # size overflow
    (dict(ws=P + 2**31 + 16, wsb=60416), ALIGN),           # workspace needs 256-byte alignment
    (dict(ws=P + 2**24, wsb=60416), INVALID),               # workspace overlaps k
    (dict(ws=P + 2**31, wsb=60415), WSERR),                 # bf16 workspace below one block
    (dict(ws=P + 2**31, wsb=0), WSERR),                     # a non-NULL workspace of zero bytes
    (dict(ws=P + 2**31, wsb=60416, T=65), WSERR),           # two chunks need two blocks
])
def test_chunk_fwd_rejects(lib, kw, code):
    assert chunk(lib, **kw) == code


def test_chunk_fwd_noop_and_in_place_accepted_shapes(lib):
    # B*H == 0 returns before any launch, even with NULL pointers
    assert lib.kda_chunk_fwd(None, None, None, None, None, None, None, None,
                             0, 64, 4, 128, 128, BF16, None, 0, None) == OK
    assert lib.kda_chunk_fwd(None, None, None, None, None, None, None, None,
                             3, 64, 0, 128, 128, F32, None, 0, None) == OK
    # T == 0 with S_T == NULL: nothing to do
    assert chunk(lib, q=None, k=None, v=None, g=None, beta=None, o=None, ST=None, T=0) == OK


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), INVALID), (dict(S=None), INVALID), (dict(o=None), INVALID),
    (dict(N=-1), INVALID), (dict(dk=32), UNSUP), (dict(dt=3), UNSUP),
    (dict(S=P + 2**28 + 4), ALIGN), (dict(v=P + 2**25 + 2), ALIGN),
    (dict(o=P + 2**28), INVALID),   # o inside S
    (dict(S=P), INVALID),           # S overlaps q
    (dict(N=2**31 - 1, H=4), UNSUP),
])
def test_recurrent_step_rejects(lib, kw, code):
    assert step(lib, **kw) == code


def test_block_and_scan_workspace_queries(lib):
    assert lib.kda_chunk_fwd_block_bytes() == 60416
    f = lib.kda_chunk_fwd_scan_workspace_size
    assert f(1, 65536, 32, 128, 128, BF16) == 32 * 1024 * 60416
    assert f(2, 65, 3, 128, 128, BF16) == 6 * 2 * 60416
    assert f(1, 64, 1, 128, 128, F32) == 0            # fp32 uses no workspace
    assert f(1, 0, 1, 128, 128, BF16) == 0 and f(1, 64, 1, 64, 128, BF16) == 0


def steps(lib, q=P, k=P + 2**24, v=P + 2**25, g=P + 2**26, gate=0, beta=P + 2**27, accept=None, S=P + 2**28,
          o=P + 2**29, N=2, m=3, H=4, dk=128, dv=128, dt=BF16):
    return lib.kda_recurrent_steps(q, k, v, g, gate, beta, accept, S, o, N, m, H, dk, dv, dt, None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), INVALID), (dict(S=None), INVALID), (dict(N=-1), INVALID), (dict(m=-1), INVALID),
    (dict(dk=64), UNSUP), (dict(dt=5), UNSUP), (dict(gate=7), UNSUP),
    (dict(gate=2), INVALID),                    # no gate: log_alpha must be NULL
    (dict(accept=P + 2**30 + 2), ALIGN), (dict(o=P + 2**29 + 8), ALIGN),
    (dict(S=P + 2**24 + 64), INVALID),          # S overlaps k
    (dict(o=P + 2**28 + 1024), INVALID),        # o inside S
    (dict(accept=P + 2**28 + 64), INVALID),     # accept inside S (which is written)
])
def test_recurrent_steps_rejects(lib, kw, code):
    assert steps(lib, **kw) == code


def test_recurrent_steps_noop_shapes(lib):
    assert steps(lib, m=0, q=None, k=None, v=None, g=None, beta=None, S=None, o=None) == OK
    assert steps(lib, N=0, q=None, k=None, v=None, g=None, beta=None, S=None, o=None) == OK


def test_noalloc_rejects_on_the_host(lib):
    # the scratch array holds 128 MiB: the 32-head 65536-token prefill needs
    # 2.4 GB of operand blocks and is rejected before any HIP call
    assert lib.kda_chunk_fwd_noalloc(P, P + 2**24, P + 2**25, P + 2**26, 0, P + 2**27, None, P + 2**28,
                                     P + 2**29, 1, 65536, 32, 128, 128, BF16, None) == WSERR
    # argument errors as for kda_chunk_fwd_gated (checked before the scratch lookup
    # only when no scratch is needed: fused-kernel shapes)
    assert lib.kda_chunk_fwd_noalloc(None, P, P, P, 0, P, None, P, P, 2, 100, 64, 128, 128, BF16, None) == INVALID
    assert lib.kda_chunk_fwd_noalloc(P, P, P, P, 0, P, None, P, P, 1, 64, 1, 64, 128, BF16, None) == UNSUP


def test_fp32_ignores_a_small_workspace(lib):
    # the workspace only serves the bf16 two-kernel schedule; validation of an
    # fp32 call then fails on the (bogus) data pointers' overlap, not on size
    assert chunk(lib, dt=F32, ws=P + 2**31, wsb=16, o=P) == INVALID


def test_workspace_size_query(lib):
    f = lib.kda_chunk_fwd_workspace_size
    # few heads, bf16: two-kernel schedule, one 60,416-byte block per chunk
    # 24 to 48 heads (a multiple of 8): prep and scan pipelined in one launch,
    # one int32 ready flag per block and 8 arrival counters after the blocks
    assert f(1, 65536, 32, 128, 128, BF16) == 32 * 1024 * 60416 + (32 * 1024 + 8) * 4
    assert f(2, 1000, 20, 128, 128, BF16) == 40 * 16 * 60416 + (40 * 16 + 8) * 4
    assert f(1, 1000, 36, 128, 128, BF16) == 36 * 16 * 60416            # not a multiple of 8: one pass
    assert f(1, 64, 32, 128, 128, BF16) == 0                            # one chunk: fused kernel
    assert f(1, 100, 3, 128, 128, BF16) == 3 * 2 * 60416
    # 16 heads or fewer over enough chunks: the state scan runs in nseg
    # segments: fp32 summaries [nseg - 1][128][256], entry states [nseg][128][128]
    SEG = lambda n: (3 * (n - 1) + 1) * 128 * 128 * 4
    assert f(1, 32768, 16, 128, 128, BF16) == 16 * 512 * 60416 + 16 * SEG(4)      # 4 segments
    assert f(1, 4096, 1, 128, 128, BF16) == 64 * 60416 + SEG(16)                  # 16 segments
    assert f(2, 1300, 4, 128, 128, BF16) == 8 * 21 * 60416 + 8 * SEG(7)           # 7 segments of 3 chunks
    assert f(1, 256, 16, 128, 128, BF16) == 16 * 4 * 60416 + 16 * SEG(2)          # 2 segments of 2 chunks
    # many heads, fp32, tiny T or bad arguments: fused kernel, no workspace
    assert f(8, 4096, 16, 128, 128, BF16) == 0
    assert f(1, 256, 1, 128, 128, F32) == 0
    assert f(1, 64, 1, 128, 128, BF16) == 0
    assert f(1, 100, 3, 64, 128, BF16) == 0 and f(-1, 100, 3, 128, 128, BF16) == 0
    # T = 0 needs no workspace: any size is accepted
    assert chunk(lib, ws=P + 2**31, wsb=100, T=0, q=None, k=None, v=None, g=None, beta=None,
                 o=None, ST=None) == OK


def test_recurrent_step_empty_is_noop(lib):
    assert lib.kda_recurrent_step(None, None, None, None, None, None, None,
                                  0, 32, 128, 128, BF16, None) == OK


def test_binding_raises_without_gpu_tensors():
    torch = pytest.importorskip("torch")
    x = torch.zeros(1, 4, 1, 128)
    with pytest.raises(ValueError):
        kda.chunk_fwd(x, x, x[..., :64], x, torch.zeros(1, 4, 1))


# ----------------------------------------------------------------- layer
LAYER_W = 11                                   # weight pointers of kda_layer_fwd


def layer(lib, x=P, ws=P + 2**32, wsb=2**31, y=P + 2**33, B=1, T=64, dm=256, H=2, rank=64,
          w=None):
    w = list(w) if w is not None else [P + 2**34 + i * 2**26 for i in range(LAYER_W)]
    return lib.kda_layer_fwd(x, *w, y, B, T, dm, H, rank, ws, wsb, None)


def test_layer_workspace_layout(lib):
    offs = (ctypes.c_size_t * 10)()
    B, T, dm, H, r = 1, 32768, 2048, 16, 128
    total = lib.kda_layer_workspace_layout(B, T, dm, H, r, offs)
    R, hd = B * T, H * 128
    sizes = [R * 4 * hd * 2, R * 144 * 4, R * hd * 2, R * hd * 2, R * hd * 2, R * hd * 4,
             R * H * 2, R * hd * 2, R * hd * 2, H * 512 * 60416 + H * 10 * 128 * 128 * 4]
    assert list(offs)[0] == 0
    for i in range(9):
        assert offs[i + 1] - offs[i] == (sizes[i] + 255) // 256 * 256
        assert offs[i] % 256 == 0
    assert total == offs[9] + sizes[9]
    # many heads: the fused chunk kernel runs and needs no chunk scratch
    total8 = lib.kda_layer_workspace_layout(8, 4096, 2048, 16, 128, offs)
    assert total8 == offs[9]
    assert lib.kda_layer_workspace_layout(1, 64, 100, 2, 64, None) == 0     # d_model % 64
    assert lib.kda_layer_workspace_layout(1, 64, 256, 2, 96, None) == 0     # rank % 64
    assert lib.kda_layer_workspace_layout(1, 2**20, 2048, 16, 128, None) == 0  # too large


@pytest.mark.parametrize("kw,code", [
    (dict(x=None), INVALID), (dict(y=None), INVALID), (dict(ws=None), INVALID),
    (dict(wsb=1000), WSERR),                    # workspace too small
    (dict(B=-1), INVALID), (dict(H=0), INVALID), (dict(rank=0), INVALID),
    (dict(dm=100), UNSUP), (dict(rank=96), UNSUP), (dict(T=2**20, dm=2048, H=16), UNSUP),
    (dict(x=P + 8), ALIGN), (dict(ws=P + 2**32 + 128), ALIGN),
    (dict(w=[None] + [P + 2**34 + i * 2**26 for i in range(1, LAYER_W)]), INVALID),
    (dict(w=[P + 2**34 + i * 2**26 + (4 if i == 5 else 0) for i in range(LAYER_W)]), ALIGN),
    (dict(y=P), INVALID),                       # y overlaps x
    (dict(y=P + 2**32 + 4096), INVALID),        # y inside the workspace
    (dict(ws=P + 2**34), INVALID),              # workspace overlaps W_q
])
def test_layer_fwd_rejects(lib, kw, code):
    assert layer(lib, **kw) == code


def test_layer_fwd_empty_is_noop(lib):
    assert layer(lib, T=0, x=None, y=None, ws=None, wsb=0) == OK


# ------------------------------------------------------------ backward pass
BWD_UNIT = 235520   # workspace bytes per (batch, head, 64-token chunk)


def bwd(lib, q=P, k=P + 2**24, v=P + 2**25, g=P + 2**26, beta=P + 2**27, S0=None,
        do=P + 2**28, dST=None, dq=P + 2**29, dk=P + 2**30, dv=P + 2**31, dg=P + 2**32,
        dbeta=P + 2**33, dS0=None, B=1, T=64, H=1, kd=128, vd=128, dt=BF16,
        ws=P + 2**34, wsb=BWD_UNIT):
    return lib.kda_chunk_bwd(q, k, v, g, beta, S0, do, dST, dq, dk, dv, dg, dbeta, dS0,
                             B, T, H, kd, vd, dt, ws, wsb, None)


def test_bwd_workspace_size(lib):
    f = lib.kda_chunk_bwd_workspace_size
    assert f(8, 4096, 16, 128, 128, BF16) == 8 * 16 * 64 * BWD_UNIT
    assert f(1, 65, 3, 128, 128, BF16) == 3 * 2 * BWD_UNIT
    assert f(1, 0, 3, 128, 128, BF16) == 0
    assert f(1, 64, 1, 128, 128, F32) == 0 and f(1, 64, 1, 64, 128, BF16) == 0
    assert f(-1, 64, 1, 128, 128, BF16) == 0


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), INVALID), (dict(do=None), INVALID), (dict(dq=None), INVALID),
    (dict(dg=None), INVALID), (dict(dbeta=None), INVALID), (dict(ws=None), INVALID),
    (dict(B=-1), INVALID), (dict(T=-3), INVALID),
    (dict(dt=F32), UNSUP), (dict(dt=5), UNSUP), (dict(kd=64), UNSUP), (dict(vd=32), UNSUP),
    (dict(q=P + 2), ALIGN), (dict(dk=P + 2**30 + 8), ALIGN), (dict(dbeta=P + 2**33 + 1), ALIGN),
    (dict(ws=P + 2**34 + 16), ALIGN), (dict(dS0=P + 2**35 + 4), ALIGN),
    (dict(wsb=BWD_UNIT - 1), WSERR),             # workspace too small
    (dict(dq=P + 2**24), INVALID),               # dq overlaps k
    (dict(dv=P + 2**29 + 64), INVALID),          # dv overlaps dq
    (dict(ws=P + 2**26), INVALID),               # workspace overlaps g
    (dict(dS0=P + 2**35, dST=P + 2**35 + 16), INVALID),   # dS0 overlaps dS_T
    (dict(B=2**30, H=2**30), UNSUP),             # size overflow
])
def test_chunk_bwd_rejects(lib, kw, code):
    assert bwd(lib, **kw) == code


def bwd_g(lib, gate, g=P + 2**26, dg=P + 2**32, **kw):
    a = dict(q=P, k=P + 2**24, v=P + 2**25, beta=P + 2**27, S0=None, do=P + 2**28, dST=None,
             dq=P + 2**29, dk=P + 2**30, dv=P + 2**31, dbeta=P + 2**33, dS0=None, B=1, T=64, H=1,
             kd=128, vd=128, dt=BF16, ws=P + 2**34, wsb=BWD_UNIT)
    a.update(kw)
    return lib.kda_chunk_bwd_gated(a["q"], a["k"], a["v"], g, gate, a["beta"], a["S0"], a["do"], a["dST"],
                                   a["dq"], a["dk"], a["dv"], dg, a["dbeta"], a["dS0"], a["B"], a["T"],
                                   a["H"], a["kd"], a["vd"], a["dt"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize("gate,kw,code", [
    (3, {}, UNSUP), (-1, {}, UNSUP),
    (2, dict(g=P + 2**26, dg=None), INVALID),          # no gate: g must be NULL
    (2, dict(g=None, dg=P + 2**32), INVALID),          # ... and so must dg
    (2, dict(g=None, dg=None, ws=P + 2**34 + 16), ALIGN),   # NULL g, dg accepted: next check fails
    (0, dict(g=None, dg=None, ws=P + 2**34 + 16), INVALID),  # per channel: g required
    (1, dict(g=None), INVALID), (1, dict(dg=None), INVALID),
    (1, dict(g=P + 2**26 + 2), ALIGN),                 # per head: 4-byte alignment
    (0, dict(g=P + 2**26 + 4), ALIGN),                 # per channel: 16-byte alignment
    (1, dict(dg=P + 2**26 + 128), INVALID),            # dg overlaps g ([1, 64, 1] fp32 = 256 B)
    (1, dict(dg=P + 2**26 + 252), INVALID),            # dg overlaps g's last element
])
def test_chunk_bwd_gated_rejects(lib, gate, kw, code):
    assert bwd_g(lib, gate, **kw) == code


def test_chunk_bwd_noop(lib):
    # B*H == 0 returns before any launch, even with NULL pointers
    assert lib.kda_chunk_bwd(*([None] * 14), 0, 64, 4, 128, 128, BF16, None, 0, None) == OK
    # T == 0 without dS0: nothing to write
    assert lib.kda_chunk_bwd(*([None] * 14), 2, 0, 4, 128, 128, BF16, None, 0, None) == OK


# ------------------------------------------------------------- gate variants
GATE_CHANNEL, GATE_HEAD, GATE_NONE = 0, 1, 2


def chunk_g(lib, gate, g=P + 2**26, T=64, **kw):
    a = dict(q=P, k=P + 2**24, v=P + 2**25, beta=P + 2**27, S0=None, o=P + 2**28, ST=P + 2**29,
             B=1, H=1, dk=128, dv=128, dt=BF16, ws=None, wsb=0)
    a.update(kw)
    return lib.kda_chunk_fwd_gated(a["q"], a["k"], a["v"], g, gate, a["beta"], a["S0"], a["o"], a["ST"],
                                   a["B"], T, a["H"], a["dk"], a["dv"], a["dt"], a["ws"], a["wsb"], None)


def step_g(lib, gate, g=P + 2**26, **kw):
    a = dict(q=P, k=P + 2**24, v=P + 2**25, beta=P + 2**27, S=P + 2**28, o=P + 2**29, N=1, H=1, dt=BF16)
    a.update(kw)
    return lib.kda_recurrent_step_gated(a["q"], a["k"], a["v"], g, gate, a["beta"], a["S"], a["o"],
                                        a["N"], a["H"], 128, 128, a["dt"], None)


def test_gated_entry_points_reject(lib):
    assert chunk_g(lib, 3) == UNSUP and chunk_g(lib, -1) == UNSUP
    assert step_g(lib, 7) == UNSUP
    assert chunk_g(lib, GATE_NONE) == INVALID          # no decay: log_alpha must be NULL
    assert step_g(lib, GATE_NONE) == INVALID
    assert chunk_g(lib, GATE_HEAD, g=P + 2**26 + 2) == ALIGN   # per-head gate: 4-byte aligned
    assert chunk_g(lib, GATE_CHANNEL, g=P + 2**26 + 4) == ALIGN
    assert chunk_g(lib, GATE_HEAD, g=None) == INVALID
    assert chunk_g(lib, GATE_HEAD, g=P + 2**28 + 4) == INVALID        # gate overlaps o
    # zero heads: no-op for every gate
    assert chunk_g(lib, GATE_HEAD, H=0) == OK and chunk_g(lib, GATE_NONE, g=None, H=0) == OK
    assert step_g(lib, GATE_HEAD, N=0) == OK
    # T = 0 without S_T touches nothing, whatever the gate
    assert chunk_g(lib, GATE_NONE, g=None, T=0, q=None, k=None, v=None, beta=None, o=None, ST=None) == OK


# ------------------------------------------------------ packed sequences
def varlen(lib, q=P, k=P + 2**24, v=P + 2**25, g=P + 2**26, gate=0, beta=P + 2**27, cu=P + 2**30,
           ns=2, S0=None, o=P + 2**28, ST=P + 2**29, total=100, H=1, dt=BF16):
    return lib.kda_chunk_fwd_varlen(q, k, v, g, gate, beta, cu, ns, S0, o, ST, total, H, 128, 128, dt, None)


@pytest.mark.parametrize("kw,code", [
    (dict(cu=None), INVALID), (dict(cu=P + 2**30 + 2), ALIGN), (dict(ns=-1), INVALID),
    (dict(total=-5), INVALID), (dict(gate=5), UNSUP), (dict(dt=9), UNSUP),
    (dict(gate=2), INVALID),                     # no decay: log_alpha must be NULL
    (dict(o=P + 2**30), INVALID),                # o overlaps cu_seqlens
    (dict(ST=P + 2**30 - 64), INVALID),          # S_T overlaps cu_seqlens
    (dict(q=P + 8), ALIGN), (dict(o=None), INVALID),
])
def test_varlen_rejects(lib, kw, code):
    assert varlen(lib, **kw) == code


def test_varlen_noop(lib):
    assert varlen(lib, ns=0) == OK and varlen(lib, H=0) == OK


# ------------------------------------------------- full-attention decode
def mqa(lib, q=P, c=P + 2**24, o=P + 2**34, B=1, T=100, H=32, D=512, ws=P + 2**35, wsb=1 << 20):
    return lib.kda_mqa_decode(q, c, o, B, T, H, D, 0.04, ws, wsb, None)


def test_mqa_workspace_size(lib):
    f = lib.kda_mqa_decode_workspace_size
    assert f(1, 1 << 20, 32, 512) == 256 * 32 * 512 * 4 + 256 * 32 * 2 * 4
    assert f(2, 100, 16, 512) == 2 * 16 * 512 * 4 + 256
    assert f(1, 0, 32, 512) == 0 and f(1, 10, 24, 512) == 0 and f(1, 10, 32, 256) == 0


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), INVALID), (dict(c=None), INVALID), (dict(o=None), INVALID), (dict(ws=None), INVALID),
    (dict(B=-1), INVALID), (dict(T=0), INVALID), (dict(H=24), UNSUP), (dict(D=128), UNSUP),
    (dict(T=(1 << 22) + 1), UNSUP),
    (dict(q=P + 4), ALIGN), (dict(ws=P + 2**35 + 64), ALIGN), (dict(wsb=100), WSERR),
    (dict(o=P + 2**24 + 64), INVALID),           # o inside the cache
    (dict(ws=P), INVALID),                       # workspace overlaps q
])
def test_mqa_rejects(lib, kw, code):
    assert mqa(lib, **kw) == code


def test_mqa_noop(lib):
    assert lib.kda_mqa_decode(None, None, None, 0, 100, 32, 512, 0.1, None, 0, None) == OK


# ------------------------------------------------------ DPLR comparison path
DPLR_UNIT = 72704 + 32768   # workspace bytes per (batch, head, 64-token chunk), plus 512 per head-token and 256


def dplr(lib, q=P, k=P + 2**24, v=P + 2**25, a=P + 2**26, b=P + 2**27, g=P + 2**28, S0=None,
         o=P + 2**29, ST=None, B=1, T=64, H=1, kd=128, vd=128, dt=BF16, ws=P + 2**34, wsb=None):
    if wsb is None:
        wsb = lib.kda_dplr_chunk_fwd_workspace_size(B, T, H, kd, vd, dt)
    return lib.kda_dplr_chunk_fwd(q, k, v, a, b, g, S0, o, ST, B, T, H, kd, vd, dt, ws, wsb, None)


def test_dplr_workspace_size(lib):
    f = lib.kda_dplr_chunk_fwd_workspace_size
    assert f(1, 64, 1, 128, 128, BF16) == DPLR_UNIT + 2 * 64 * 256 + 256   # + one sink row
    assert f(8, 4096, 16, 128, 128, BF16) == 8 * 16 * 64 * (DPLR_UNIT + 2 * 64 * 256) + 256
    assert f(1, 65, 1, 128, 128, BF16) == 2 * DPLR_UNIT + 2 * 65 * 256 + 256    # U0, O0: one row per token
    assert f(1, 64, 1, 128, 128, F32) == 0 and f(1, 64, 1, 64, 128, BF16) == 0 and f(-1, 64, 1, 128, 128, BF16) == 0


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), INVALID), (dict(a=None), INVALID), (dict(b=None), INVALID), (dict(g=None), INVALID),
    (dict(o=None), INVALID), (dict(ws=None), INVALID), (dict(B=-1), INVALID), (dict(T=-1), INVALID),
    (dict(dt=F32), UNSUP), (dict(kd=64), UNSUP), (dict(vd=256), UNSUP),
    (dict(a=P + 2**26 + 8), ALIGN), (dict(g=P + 2**28 + 4), ALIGN), (dict(ws=P + 2**34 + 16), ALIGN),
    (dict(wsb=1000), WSERR),                     # workspace too small
    (dict(o=P + 2**27 + 64), INVALID),           # o overlaps b
    (dict(ws=P + 2**28), INVALID),               # workspace overlaps the log-decay
    (dict(S0=P + 2**35, ST=P + 2**35 + 16), INVALID),   # S_T overlaps S0 partially
    (dict(ST=P + 2**29), INVALID),               # S_T overlaps o
    (dict(B=2**30, H=2**30), UNSUP),             # size overflow
])
def test_dplr_rejects(lib, kw, code):
    assert dplr(lib, **kw) == code


def test_dplr_noop(lib):
    assert lib.kda_dplr_chunk_fwd(*([None] * 9), 0, 64, 4, 128, 128, BF16, None, 0, None) == OK
    assert lib.kda_dplr_chunk_fwd(*([None] * 9), 2, 0, 4, 128, 128, BF16, None, 0, None) == OK
