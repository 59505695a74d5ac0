"""GPU parity of one whole attention layer's decode step (DecodeLayer: cache write -> query side
-> absorbed attention -> W_UV -> W_O) against the oracle composed from the same steps.

The oracle side: the new cache row from oracle.cache_write (stored as its own bf16 rounding), the
query side from oracle.query with c_q, q_C and q_R held in bf16 the way the layer stores them,
the explicit-K/V decode of oracle.decode over the cache rows 0 .. pos (inclusive), then
oracle.output.out_proj.  Bar: relative L2 <= 1e-2 (the bf16 path), and the written cache rows
within one bf16 step of the exact values.  Two V3-shape batches: 2 sequences (GEMV projections)
and 5 (the MFMA path for the K = 1536 projection), ragged lengths including an empty cache.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import oracle.output as oo
import oracle.query as oq
from mla_latent_kv_attn_amd import ops
from mla_latent_kv_attn_amd.layer import DecodeLayer
from oracle import decode_bf16, relative_l2
from oracle.cache_write import cache_row, encode_bf16
from tests._helpers import custom_inputs
from workloads.layer import make_layer_inputs

pytestmark = pytest.mark.gpu

H, D_H, D_C, D_R = 128, 128, 512, 64


def _dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def _bits(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def _held(x):
    """bf16 storage of an exact value (the oracle's own rounding)."""
    return decode_bf16(encode_bf16(x))


def _oracle_layer(inp):
    W = {k: decode_bf16(v) for k, v in inp.weights.items()}
    h = decode_bf16(inp.h)
    pos = inp.pos
    row = cache_row(h, W["W_DKV"], W["W_KR"], pos)
    c_q = _held(oq.q_down(W["W_DQ"], h))
    q_C, q_R = oq.q_up(W["W_UQ"], W["W_QR"], c_q, pos, H)
    q_C, q_R = _held(q_C), _held(q_R)
    C_rows, R_rows = [], []
    for b in range(len(pos)):
        L = int(pos[b])
        C_rows.append(np.concatenate([decode_bf16(inp.latent[b, :L]), decode_bf16(row["c_bf16"][b:b + 1])]))
        R_rows.append(np.concatenate([decode_bf16(inp.rope[b, :L]), decode_bf16(row["k_R_bf16"][b:b + 1])]))
    ref = oracle.decode(custom_inputs(q_C, q_R, W["W_UK"], W["W_UV"], C_rows, R_rows), want_diag=False)
    return oo.out_proj(W["W_O"], ref["o"]), row


@pytest.mark.parametrize("lens", [[0, 300], [5, 64, 131, 2, 257]])
def test_decode_layer_matches_oracle(lens):
    print(f"DecodeLayer V3 lens={lens}", flush=True)
    cap = 320
    inp = make_layer_inputs(lens, cap)
    B = len(lens)
    weights = {k: _dev(v) for k, v in inp.weights.items()}
    lat, rope = _dev(inp.latent), _dev(inp.rope)
    cache = ops.Cache.split(lat, rope)
    pos = torch.from_numpy(inp.pos).cuda()
    seq_lens = torch.from_numpy(inp.pos + 1).cuda()
    layer = DecodeLayer(weights, cache, B, max_len=cap)
    y = layer(_dev(inp.h), pos, seq_lens)
    torch.cuda.synchronize()
    y_ref, row = _oracle_layer(inp)
    err = relative_l2(y.cpu().numpy().astype(np.float64), y_ref)
    assert err <= 1e-2, err
    # the new rows are written where they belong, within one bf16 step of the exact values
    lat_h, rope_h = _bits(lat), _bits(rope)
    for b in range(B):
        p = int(inp.pos[b])
        for got, exact in ((lat_h[b, p], row["c"][b]), (rope_h[b, p], row["k_R"][b])):
            g = decode_bf16(got)
            step = np.exp2(np.floor(np.log2(np.maximum(np.abs(exact), 2.0 ** -126))) - 7)
            assert np.all(np.abs(g - exact) <= step * 1.0001 + 1e-6)
        assert np.array_equal(lat_h[b, :p], inp.latent[b, :p]) and np.array_equal(lat_h[b, p + 1:], inp.latent[b, p + 1:])


def test_decode_layer_graph_replays_match_eager():
    # the whole layer captured once in a HIP graph; several replays with eager work and
    # synchronisations between them, each checked against the eager result (bitwise: same kernels,
    # same launch shapes, deterministic reductions)
    print("DecodeLayer graph replays", flush=True)
    lens = [17, 200, 64]
    cap = 256
    inp = make_layer_inputs(lens, cap, seed=53)
    B = len(lens)
    weights = {k: _dev(v) for k, v in inp.weights.items()}
    lat, rope = _dev(inp.latent), _dev(inp.rope)
    cache = ops.Cache.split(lat, rope)
    pos = torch.from_numpy(inp.pos).cuda()
    seq_lens = torch.from_numpy(inp.pos + 1).cuda()
    h = _dev(inp.h)
    layer = DecodeLayer(weights, cache, B, max_len=cap)
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        eager = layer(h, pos, seq_lens, stream=stream).clone()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        layer(h, pos, seq_lens, stream=stream)
    for rep in range(3):
        layer.y.fill_(float("nan"))
        junk = torch.randn(1 << 20, device="cuda").sum()      # eager work between replays
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            g.replay()
        torch.cuda.synchronize()
        assert torch.equal(layer.y, eager), f"replay {rep} differs from the eager layer"
        assert torch.isfinite(junk)


def _within_bf16_step(a_bits, b_bits):
    ga, gb = decode_bf16(a_bits), decode_bf16(b_bits)
    same = np.isnan(ga) & np.isnan(gb)
    step = np.exp2(np.floor(np.log2(np.maximum(np.abs(np.nan_to_num(gb)), 2.0 ** -126))) - 7)
    return np.all(same | (np.abs(ga - gb) <= step * 1.0001))


@pytest.mark.parametrize("B", [1, 3, 8, 12, 64])
def test_query_proj_append_matches_separate_calls(B):
    # one pass over [W_DQ; W_DKV; W_KR] against mla_cache_append + mla_query_proj on a copy of the
    # cache: bitwise up to 8 tokens (the same projection kernel per row); beyond, the fused pass
    # splits K into other chunks than the separate calls (sums in another order): c_q and the cache
    # row within one bf16 step, q_C / q_R (from that c_q) within relative L2 1e-3
    print(f"mla_query_proj_append B={B}", flush=True)
    rng = np.random.default_rng(60 + B)
    lens = rng.integers(0, 120, size=B)
    cap = 128
    inp = make_layer_inputs(lens, cap, seed=61 + B)
    w = {k: _dev(v) for k, v in inp.weights.items()}
    h = _dev(inp.h)
    pos = torch.from_numpy(inp.pos).cuda()
    lat_a, rope_a = _dev(inp.latent), _dev(inp.rope)
    lat_b, rope_b = lat_a.clone(), rope_a.clone()
    fused = ops.mla_query_proj_append(h, w["W_DQ"], w["W_UQ"], w["W_QR"], w["W_DKV"], w["W_KR"], pos,
                                      ops.Cache.split(lat_a, rope_a), H)
    ops.mla_cache_append(h, w["W_DKV"], w["W_KR"], pos, ops.Cache.split(lat_b, rope_b))
    sep = ops.mla_query_proj(h, w["W_DQ"], w["W_UQ"], w["W_QR"], pos, H)
    torch.cuda.synchronize()
    if B <= 8:
        for x, y in zip(fused, sep):
            assert np.array_equal(_bits(x), _bits(y))
        assert np.array_equal(_bits(lat_a), _bits(lat_b)) and np.array_equal(_bits(rope_a), _bits(rope_b))
    else:
        assert _within_bf16_step(_bits(fused[0]), _bits(sep[0]))
        for x, y in zip(fused[1:], sep[1:]):
            assert relative_l2(decode_bf16(_bits(x)).astype(np.float64), decode_bf16(_bits(y)).astype(np.float64)) <= 1e-3
        for a_, b_ in ((lat_a, lat_b), (rope_a, rope_b)):
            assert _within_bf16_step(_bits(a_), _bits(b_))
