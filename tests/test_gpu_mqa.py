"""GPU parity of the full-attention decode step (kda_mqa_decode through the C
ABI: MQA over a shared 512-wide latent, the inference form of a NoPE MLA
layer) against the fp64 oracle, on every output element at sizes that span
several 64-token tiles, 4096-token splits and ragged tails, and on sampled
heads of a 1M-token cache."""
import math

import pytest
import torch

import gated_delta_rule_32_amd as kda
from gated_delta_rule_32_amd import inputs
from oracle import mqa_ref
from tests.kda_testutil import TOL, max_rel_err

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.mark.parametrize("H", [16, 32])
@pytest.mark.parametrize("T", [1, 63, 64, 65, 4096, 4097, 10000])
def test_mqa_decode_matches_oracle(H, T):
    print(f"mqa decode H={H} T={T}", flush=True)
    q, c = inputs.mqa_inputs(2, T, H, seed=T + H)
    scale = 1.0 / math.sqrt(512)
    o = kda.mqa_decode(q.to(DEV), c.to(DEV), scale)
    torch.cuda.synchronize()
    ref = mqa_ref.decode(q, c, scale)
    err = max_rel_err(o, ref)
    print(f"  err {err:.3e}", flush=True)
    assert err <= TOL["bfloat16"]


def test_mqa_decode_peaked_softmax():
    """A large scale makes each head's weights nearly one-hot: the running
    maximum must be carried correctly across tiles and splits."""
    q, c = inputs.mqa_inputs(1, 9000, 32, seed=3)
    o = kda.mqa_decode(q.to(DEV), c.to(DEV), 0.5)
    torch.cuda.synchronize()
    err = max_rel_err(o, mqa_ref.decode(q, c, 0.5))
    print(f"  peaked: err {err:.3e}", flush=True)
    assert err <= TOL["bfloat16"]


def test_mqa_decode_1m_tokens_sampled_heads():
    """The benchmarked shape, B = 1, T = 2^20, H = 32, D = 512: heads 0, 13 and
    31 against the oracle."""
    cfg = inputs.MQA_CONFIG
    q, c = inputs.mqa_inputs(cfg["B"], cfg["T"], cfg["H"], seed=cfg["seed"], device=DEV)
    scale = 1.0 / math.sqrt(512)
    o = kda.mqa_decode(q, c, scale)
    torch.cuda.synchronize()
    heads = [0, 13, 31]
    ref = mqa_ref.decode(q.cpu(), c.cpu(), scale, heads=heads)
    err = max_rel_err(o[:, heads], ref)
    print(f"  1M tokens, heads {heads}: err {err:.3e}", flush=True)
    assert err <= TOL["bfloat16"]
