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
OK, INVALID, UNSUP, ALIGN = 0, -1, -2, -3
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
    assert set(names) == {"kda_chunk_fwd", "kda_chunk_fwd_workspace_size", "kda_recurrent_step",
                          "kda_status_string", "kda_version"}
    for n in names:
        assert hasattr(lib, n), n
    assert set(_binding.SIGNATURES) == set(names)


def test_status_strings(lib):
    for code in (OK, INVALID, UNSUP, ALIGN, -4, 12345):
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
    (dict(ws=P + 2**31 + 16, wsb=66048), ALIGN),           # workspace needs 256-byte alignment
    (dict(ws=P + 2**24, wsb=66048), INVALID),               # workspace overlaps k
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


def test_workspace_size_query(lib):
    f = lib.kda_chunk_fwd_workspace_size
    # few heads, bf16: two-kernel schedule, one 66,048-byte block per chunk
    assert f(1, 65536, 32, 128, 128, BF16) == 32 * 1024 * 66048
    assert f(1, 32768, 16, 128, 128, BF16) == 16 * 512 * 66048
    assert f(1, 100, 3, 128, 128, BF16) == 3 * 2 * 66048
    # many heads, fp32, tiny T or bad arguments: fused kernel, no workspace
    assert f(8, 4096, 16, 128, 128, BF16) == 0
    assert f(1, 256, 1, 128, 128, F32) == 0
    assert f(1, 64, 1, 128, 128, BF16) == 0
    assert f(1, 100, 3, 64, 128, BF16) == 0 and f(-1, 100, 3, 128, 128, BF16) == 0
    # a workspace too small is simply not used (fused kernel): no error
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
