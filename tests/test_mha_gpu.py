"""GPU parity of the same-dimension MHA comparison path (mla_mha_decode) against the oracle's
plain softmax attention (oracle.attend, pinned in tests/test_oracle_pins.py) on the same explicit
bf16 K/V.  Arithmetic is fp32 on exactly representable inputs: relative L2 <= 2e-5 per head.
Padding rows hold NaN, so a read past a sequence's end shows up as a non-finite output."""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

from oracle import attend, decode_bf16, relative_l2
from workloads.mha import make_mha_inputs

pytestmark = pytest.mark.gpu


def _t(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def _run(inp, splits, max_len):
    from mla_latent_kv_attn_amd import ops
    lens = torch.from_numpy(inp.lens).cuda()
    lse = torch.empty(inp.q.shape[:2], dtype=torch.float32, device="cuda")
    print(f"[gpu] mha B={len(inp.lens)} H={inp.q.shape[1]} lens[:6]={inp.lens[:6].tolist()} splits={splits}", flush=True)
    o = ops.mla_mha_decode(_t(inp.q), _t(inp.K), _t(inp.V), lens, max_len, num_splits=splits, lse=lse)
    torch.cuda.synchronize()
    return o.cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


def _compare(inp, o, lse, heads=None):
    B, H = inp.q.shape[:2]
    scale = 1.0 / math.sqrt(192)
    assert np.all(np.isfinite(o))
    for b in range(B):
        L = int(inp.lens[b])
        for h in (heads if heads is not None else range(H)):
            K = decode_bf16(inp.K[b, h, :L])
            V = decode_bf16(inp.V[b, h, :L])
            ro, rl, _ = attend(K, V, decode_bf16(inp.q[b, h]), scale)
            if L == 0:
                assert np.all(o[b, h] == 0) and lse[b, h] == -np.inf
                continue
            assert relative_l2(o[b, h], ro) <= 2e-5, (b, h)
            assert abs(lse[b, h] - rl) <= 1e-4, (b, h)


@pytest.mark.parametrize("splits", [0, 1, 3, 7])
def test_mha_ragged(splits):
    inp = make_mha_inputs([0, 1, 63, 64, 65, 300], H=8, cap=320)
    o, lse = _run(inp, splits, 300)
    _compare(inp, o, lse)


def test_mha_v3_shape_sampled():
    """B = 1, H = 128, 4096 cached tokens (the shape of the latent path's default workload)."""
    inp = make_mha_inputs([4096], H=128, cap=4096, seed=22)
    o, lse = _run(inp, 0, 4096)
    _compare(inp, o, lse, heads=[0, 17, 64, 127])
