"""mla_decode_attn_noalloc (the workspace in the library's fixed device array) against
mla_decode_attn with a caller workspace, through the C ABI, on the GPU.

Two calls in a row, the second with a smaller input: each must give mla_decode_attn's result bit
for bit at the same split count (the same kernels over the same partition), and meet the oracle's
per-pair tolerance.  Sizes whose workspace exceeds the array are rejected before any launch.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from mla_latent_kv_attn_amd import _lib, ops
from workloads import make_inputs
from workloads.configs import WORKLOADS
from workloads.device import device_cache, to_device

pytestmark = pytest.mark.gpu


def per_pair_max(got, ref, lens):
    worst = 0.0
    B, H = got.shape[:2]
    for b in range(B):
        if lens[b] == 0:
            assert np.all(got[b] == 0.0)
            continue
        for h in range(H):
            worst = max(worst, oracle.relative_l2(got[b, h], ref[b, h]))
    return worst


def both(inp, splits):
    wl = inp.wl
    print(f"[gpu] noalloc {wl.name} B={wl.B} splits={splits} lens={inp.lens.tolist()}", flush=True)
    dev = to_device(inp)
    cache = device_cache(inp, dev)
    q_abs = ops.mla_absorb_q(dev["q_C"], dev["W_UK"])
    o_na = torch.full((wl.B, wl.H, wl.d_c), float("nan"), dtype=torch.float32, device="cuda")
    lse_na = torch.full((wl.B, wl.H), float("nan"), dtype=torch.float32, device="cuda")
    ops.mla_decode_attn_noalloc(q_abs, dev["q_R"], cache, dev["lens"], wl.n_max, o_na, lse_na, d_h=wl.d_h,
                                num_splits=splits)
    W = splits or int(_lib.lib().mla_decode_attn_noalloc_splits(wl.B, wl.H, wl.d_c, wl.n_max))
    assert W >= 1
    o_ref, lse_ref = ops.mla_decode_attn(q_abs, dev["q_R"], cache, dev["lens"], wl.n_max, d_h=wl.d_h, num_splits=W)
    torch.cuda.synchronize()
    assert torch.equal(o_na, o_ref), "o_latent differs from mla_decode_attn at the same split count"
    assert torch.equal(lse_na, lse_ref), "lse differs from mla_decode_attn at the same split count"
    ref = oracle.decode(inp)
    tol = 1e-5 if wl.dtype == "f32" else 1e-2
    err = per_pair_max(o_na.cpu().numpy().astype(np.float64), ref["o_lat"], inp.lens)
    print(f"[parity] noalloc {wl.name}: worst pair o_lat {err:.3e}", flush=True)
    assert err <= tol


def test_noalloc_two_calls_second_smaller():
    big = make_inputs(WORKLOADS[3].with_(name="na-big", B=6, n_max=1000, len_lo=1, len_hi=1000),
                      lens=np.array([1000, 31, 32, 33, 0, 517]))
    small = make_inputs(WORKLOADS[2].with_(name="na-small", B=2, n_max=130, len_lo=1, len_hi=130),
                        lens=np.array([130, 7]))
    both(big, 0)
    both(small, 0)
    both(big, 5)
    both(small, 3)


def test_noalloc_fp32_and_fp8():
    both(make_inputs(1), 0)
    both(make_inputs(WORKLOADS[5].with_(name="na-fp8", B=3, n_max=160, len_lo=1, len_hi=160),
                     lens=np.array([160, 0, 77])), 0)


def test_noalloc_rejects_sizes_beyond_the_array():
    lib = _lib.lib()
    cap = int(lib.mla_decode_attn_noalloc_max_bytes())
    assert cap == 64 << 20
    # 2048 sequences need at least 2048 partial slots of 256 KB: more than the array holds
    assert int(lib.mla_decode_attn_noalloc_splits(2048, 128, 512, 64)) == 0
    wl = WORKLOADS[2].with_(name="na-huge", B=2048, n_max=32, len_lo=1, len_hi=32)
    q_abs = torch.zeros((2048, 128, 512), dtype=torch.bfloat16, device="cuda")
    q_R = torch.zeros((2048, 128, 64), dtype=torch.bfloat16, device="cuda")
    lat = torch.zeros((2048, 32, 512), dtype=torch.bfloat16, device="cuda")
    rope = torch.zeros((2048, 32, 64), dtype=torch.bfloat16, device="cuda")
    lens = torch.ones(2048, dtype=torch.int32, device="cuda")
    o = torch.empty((2048, 128, 512), dtype=torch.float32, device="cuda")
    with pytest.raises(_lib.MlaError) as ei:
        ops.mla_decode_attn_noalloc(q_abs, q_R, ops.Cache.split(lat, rope), lens, wl.n_max, o, d_h=128)
    assert ei.value.status == _lib.MLA_ERR_WORKSPACE
    # an explicit split count whose workspace does not fit is rejected too
    with pytest.raises(_lib.MlaError) as ei:
        ops.mla_decode_attn_noalloc(q_abs[:64], q_R[:64], ops.Cache.split(lat[:64], rope[:64]), lens[:64],
                                    wl.n_max, o[:64], d_h=128, num_splits=1000)
    assert ei.value.status == _lib.MLA_ERR_WORKSPACE
