"""GPU parity of the projections around the attention core against oracle/query.py and
oracle/output.py: the query side (mla_query_proj), the offline folds (mla_fold_q, mla_fold_o),
the folded absorbed query (mla_absorb_q_folded) and the output projection (mla_out_proj).

Bars (the kernels accumulate in fp32):
  * a bf16 result rounded once from an fp32 sum: every element within one bf16 step of the exact
    value, or (where a fold's fp32 sum of 128 products may cancel) relative L2 <= 2.5e-3;
  * q_C / q_R read c_q rounded to bf16: compared with the oracle applied to its own bf16 rounding
    of the exact c_q, relative L2 <= 3e-3, and with the exact c_q, <= 1e-2;
  * fp32 results of the GEMV path (fp32 x): relative L2 <= 2e-5; of the MFMA path (x rounded to
    bf16 for the MFMA): <= 4e-3.
Sizes: the V3 shapes (D 7168, d_q 1536, H 128, d_h 128, d_c 512, d_R 64) at 1, 2, 3, 4, 8 (the GEMV
variants, and the MFMA path from 3 tokens where K < 4096), 9, 33, 100 (the MFMA tile widths,
ragged 32-token blocks) and 130 tokens (two 128-token tiles), a small non-V3 shape, positions 0
and 32767, and B = 0.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle.output as oo
import oracle.query as oq
from mla_latent_kv_attn_amd import ops
from oracle import decode_bf16, relative_l2
from oracle.cache_write import encode_bf16
from workloads.proj import make_folded_query_inputs, make_output_inputs, make_query_inputs

pytestmark = pytest.mark.gpu


def _bf16_tensor(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def _bits(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def _within_one_step(got_bits, exact, what):
    got = decode_bf16(got_bits)
    step = np.exp2(np.floor(np.log2(np.maximum(np.abs(exact), 2.0 ** -126))) - 7)
    err = np.abs(got - exact)
    bad = err > step * 1.0001 + 1e-6
    assert not bad.any(), f"{what}: {bad.sum()} values more than one bf16 step off (max err {err.max():.3g})"


def _say(msg):
    print(msg, flush=True)


# ------------------------------------------------------------------------------------ query side
@pytest.fixture(scope="module")
def v3_query():
    big = make_query_inputs(130)
    W = {k: decode_bf16(getattr(big, k)) for k in ("W_DQ", "W_UQ", "W_QR")}
    dev = {k: _bf16_tensor(getattr(big, k)) for k in ("W_DQ", "W_UQ", "W_QR", "W_UK")}
    return big, W, dev


def _check_query(inp, W, dev, B, H, rope_base=10000.0):
    h = inp.h[:B]
    pos = inp.pos[:B]
    c_q, q_C, q_R = ops.mla_query_proj(_bf16_tensor(h), dev["W_DQ"], dev["W_UQ"], dev["W_QR"],
                                       torch.from_numpy(pos).cuda(), H, rope_base)
    torch.cuda.synchronize()
    exact_cq = oq.q_down(W["W_DQ"], decode_bf16(h))
    _within_one_step(_bits(c_q), exact_cq, f"c_q B={B}")
    held = decode_bf16(encode_bf16(exact_cq))                 # c_q as the oracle itself rounds it
    ref_C, ref_R = oq.q_up(W["W_UQ"], W["W_QR"], held, pos, H, rope_base)
    got_C, got_R = decode_bf16(_bits(q_C)), decode_bf16(_bits(q_R))
    assert relative_l2(got_C, ref_C) <= 3e-3, relative_l2(got_C, ref_C)
    assert relative_l2(got_R, ref_R) <= 3e-3, relative_l2(got_R, ref_R)
    ex_C, ex_R = oq.q_up(W["W_UQ"], W["W_QR"], exact_cq, pos, H, rope_base)
    assert relative_l2(got_C, ex_C) <= 1e-2 and relative_l2(got_R, ex_R) <= 1e-2


@pytest.mark.parametrize("B", [1, 2, 3, 4, 8, 9, 33, 100, 130])
def test_query_proj_v3(v3_query, B):
    inp, W, dev = v3_query
    _say(f"mla_query_proj V3 B={B}")
    _check_query(inp, W, dev, B, 128)


def test_query_proj_extreme_positions(v3_query):
    inp, W, dev = v3_query
    _say("mla_query_proj positions 0 / 32767")
    saved = inp.pos.copy()
    try:
        for B in (4, 40):
            inp.pos[:B] = np.where(np.arange(B) % 2 == 0, 0, 32767).astype(np.int32)
            _check_query(inp, W, dev, B, 128)
    finally:
        inp.pos[:] = saved


@pytest.mark.parametrize("B", [2, 17])
def test_query_proj_small_shape(B):
    _say(f"mla_query_proj D=1024 d_q=512 H=4 d_h=32 B={B}")
    inp = make_query_inputs(B, D=1024, d_q=512, H=4, d_h=32, d_R=64, d_c=64, seed=5)
    W = {k: decode_bf16(getattr(inp, k)) for k in ("W_DQ", "W_UQ", "W_QR")}
    dev = {k: _bf16_tensor(getattr(inp, k)) for k in ("W_DQ", "W_UQ", "W_QR")}
    _check_query(inp, W, dev, B, 4, rope_base=500.0)


def test_query_proj_empty_batch(v3_query):
    _, _, dev = v3_query
    c_q = torch.full((1, 1536), 7.0, dtype=torch.bfloat16, device="cuda")
    q_C = torch.full((1, 128, 128), 7.0, dtype=torch.bfloat16, device="cuda")
    q_R = torch.full((1, 128, 64), 7.0, dtype=torch.bfloat16, device="cuda")
    h = torch.zeros(0, 7168, dtype=torch.bfloat16, device="cuda")
    ops.mla_query_proj(h, dev["W_DQ"], dev["W_UQ"], dev["W_QR"], torch.zeros(0, dtype=torch.int32, device="cuda"),
                       128, c_q=c_q[:0], q_C=q_C[:0], q_R=q_R[:0])
    torch.cuda.synchronize()
    assert bool((c_q == 7.0).all()) and bool((q_C == 7.0).all()) and bool((q_R == 7.0).all())


# ------------------------------------------------------------------------------------ query fold
def test_fold_q_small_heads_full():
    _say("mla_fold_q H=8 full")
    inp = make_query_inputs(1, H=8, seed=8)
    W_UQ, W_UK = decode_bf16(inp.W_UQ), decode_bf16(inp.W_UK)
    got = ops.mla_fold_q(_bf16_tensor(inp.W_UQ), _bf16_tensor(inp.W_UK))
    torch.cuda.synchronize()
    ref = oq.fold_q(W_UQ, W_UK)
    assert relative_l2(decode_bf16(_bits(got)), ref) <= 2.5e-3


def test_fold_q_v3_sampled_heads(v3_query):
    inp, W, dev = v3_query
    _say("mla_fold_q V3 sampled heads")
    got = ops.mla_fold_q(dev["W_UQ"], dev["W_UK"])
    torch.cuda.synchronize()
    W_UK = decode_bf16(inp.W_UK)
    for h in (0, 77, 127):
        ref = oq.fold_q(W["W_UQ"][h * 128:(h + 1) * 128], W_UK[h:h + 1])[0]
        assert relative_l2(decode_bf16(_bits(got[h])), ref) <= 2.5e-3, h


@pytest.mark.parametrize("B,out_dtype", [(1, torch.bfloat16), (4, torch.float32), (8, torch.bfloat16),
                                         (9, torch.float32), (33, torch.bfloat16)])
def test_absorb_q_folded_direct(B, out_dtype):
    # W_QK drawn directly (bf16), so the product itself is checked: fp32 sums of exact products
    _say(f"mla_absorb_q_folded direct H=32 B={B} {out_dtype}")
    c_q, W_QK = make_folded_query_inputs(B, H=32, seed=40 + B)
    got = ops.mla_absorb_q_folded(_bf16_tensor(c_q), _bf16_tensor(W_QK), out_dtype=out_dtype)
    torch.cuda.synchronize()
    ref = oq.absorb_folded(decode_bf16(W_QK), decode_bf16(c_q))
    if out_dtype == torch.bfloat16:
        _within_one_step(_bits(got), ref, f"q' B={B}")
    else:
        assert relative_l2(got.cpu().numpy().astype(np.float64), ref) <= 2e-5


def test_folded_query_matches_unfolded_oracle(v3_query):
    # end to end at the V3 shape: fold on the GPU, absorb c_q, against the oracle's
    # W_UK^T (W_UQ c_q)
    inp, W, dev = v3_query
    _say("mla_fold_q + mla_absorb_q_folded against the unfolded oracle")
    for B in (3, 12):
        c_q, _ = make_folded_query_inputs(B, H=1, seed=9)
        W_QK = ops.mla_fold_q(dev["W_UQ"], dev["W_UK"])
        got = ops.mla_absorb_q_folded(_bf16_tensor(c_q), W_QK, out_dtype=torch.float32)
        torch.cuda.synchronize()
        q_C, _ = oq.q_up(W["W_UQ"], W["W_QR"], decode_bf16(c_q), np.zeros(B, np.int32), 128)
        ref = oq.absorb(decode_bf16(inp.W_UK), q_C)
        assert relative_l2(got.cpu().numpy().astype(np.float64), ref) <= 1e-2, B
        del W_QK


# ------------------------------------------------------------------------------------ output side
@pytest.fixture(scope="module")
def v3_output():
    inp = make_output_inputs(130)
    return inp, decode_bf16(inp.W_O), _bf16_tensor(inp.W_O), _bf16_tensor(inp.W_UV)


@pytest.mark.parametrize("B", [1, 2, 5, 8, 9, 40, 100, 130])
def test_out_proj_v3(v3_output, B):
    inp, W_O, dW_O, _ = v3_output
    _say(f"mla_out_proj V3 B={B}")
    x = inp.o[:B]
    got = ops.mla_out_proj(torch.from_numpy(x).cuda(), dW_O)
    torch.cuda.synchronize()
    ref = oo.out_proj(W_O, x)
    # the GEMV (fp32 x, fp32 sums) serves W_O up to 4 tokens; from 5 (W_O has more than 32M
    # elements) the MFMA path rounds x to bf16
    tol = 2e-5 if B <= 4 else 4e-3
    assert relative_l2(got.cpu().numpy().astype(np.float64), ref) <= tol


def test_fold_o_and_folded_output(v3_output):
    inp, W_O, dW_O, dW_UV = v3_output
    _say("mla_fold_o V3 sampled heads + folded output projection")
    W_OV = ops.mla_fold_o(dW_O, dW_UV)
    torch.cuda.synchronize()
    W_UV = decode_bf16(inp.W_UV)
    for h in (0, 64, 127):
        ref = oo.fold_o(W_O[:, h * 128:(h + 1) * 128], W_UV[h:h + 1])
        assert relative_l2(decode_bf16(_bits(W_OV[:, h * 512:(h + 1) * 512])), ref) <= 2.5e-3, h
    # y = W_OV o_lat on the GPU against the oracle's W_O (W_UV o_lat) -- the two routes the
    # pages equate, the GPU's through its bf16 fold
    for B in (2, 12):
        x = inp.o_lat[:B]
        got = ops.mla_out_proj(torch.from_numpy(x).cuda(), W_OV)
        torch.cuda.synchronize()
        o = np.einsum("hik,bhk->bhi", W_UV, x.astype(np.float64))
        ref = oo.out_proj(W_O, o)
        assert relative_l2(got.cpu().numpy().astype(np.float64), ref) <= 1e-2, B
    del W_OV


def test_fold_o_small_full():
    _say("mla_fold_o D=256 H=4 full")
    inp = make_output_inputs(1, D=256, H=4, seed=3)
    got = ops.mla_fold_o(_bf16_tensor(inp.W_O), _bf16_tensor(inp.W_UV))
    torch.cuda.synchronize()
    ref = oo.fold_o(decode_bf16(inp.W_O), decode_bf16(inp.W_UV))
    assert relative_l2(decode_bf16(_bits(got)), ref) <= 2.5e-3
