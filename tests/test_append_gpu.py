"""GPU parity of mla_cache_append (the cache write) against the oracle of oracle/cache_write.py.

Each case fills the cache with a sentinel, appends one row per sequence through the C ABI and
checks (1) every byte outside the written rows is unchanged (bit-exact) and (2) the written rows
against the oracle's exact values: bf16 latent and rope within one bf16 step of the exact value
(the kernel accumulates in fp32 and rounds once), the E4M3 scale within float32 rounding of
amax/448 and every code the nearest grid value of c/s or its neighbour where c/s lies within
float32 error of a rounding boundary (the codes are a decision taken in fp32 by the kernel and in
fp64 by the oracle), at least 99.9% of them identical.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

from oracle import decode_bf16, decode_e4m3, relative_l2
from oracle.cache_write import cache_row
from workloads.append import make_append_inputs

pytestmark = pytest.mark.gpu

D, DC, DR = 7168, 512, 64
SENT16, SENT8, SENTF = 0x5A5A, 0x5A, -3.0


def _bf16_tensor(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def _bits(t: torch.Tensor) -> np.ndarray:
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def _check_bf16(got_bits, exact, what):
    got = decode_bf16(got_bits)
    step = np.exp2(np.floor(np.log2(np.maximum(np.abs(exact), 2.0 ** -126))) - 7)
    err = np.abs(got - exact)
    bad = err > step * 1.0001 + 1e-6
    assert not bad.any(), f"{what}: {bad.sum()} values more than one bf16 step off (max err {err.max():.3g})"
    assert relative_l2(got, exact) < 1e-2


def _check_fp8(codes, scale, exact, ref_codes, ref_scale, what):
    assert np.allclose(scale, ref_scale, rtol=2e-6, atol=0), f"{what}: scales"
    y = exact / ref_scale.astype(np.float64)[:, None]
    got = decode_e4m3(codes)
    a = np.abs(y)
    step = np.where(a < 2.0 ** -6, 2.0 ** -9, np.exp2(np.floor(np.log2(np.maximum(a, 2.0 ** -6))) - 3))
    assert np.all(np.abs(got - np.clip(y, -448, 448)) <= step * 1.0001), f"{what}: a code beyond the neighbouring grid value"
    same = np.mean(codes == ref_codes)
    assert same >= 0.999, f"{what}: only {same:.4%} of the codes equal the oracle's"
    assert relative_l2(decode_e4m3(codes, scale), exact) < 3e-2


def _run(cache, inp, pos, B):
    from mla_latent_kv_attn_amd import ops
    h = _bf16_tensor(inp.h)
    Wd, Wr = _bf16_tensor(inp.W_DKV), _bf16_tensor(inp.W_KR)
    p = torch.from_numpy(np.asarray(pos, dtype=np.int32)).cuda()
    print(f"[gpu] append B={B} pos[:6]={list(pos[:6])}", flush=True)
    ops.mla_cache_append(h, Wd, Wr, p, cache)
    torch.cuda.synchronize()


def _oracle(inp, pos):
    return cache_row(decode_bf16(inp.h), decode_bf16(inp.W_DKV), decode_bf16(inp.W_KR), np.asarray(pos))


@pytest.mark.parametrize("B,N,fp8", [(1, 64, False), (2, 70, False), (5, 300, False), (40, 8, False),
                                     (130, 4, False), (1, 64, True), (5, 300, True), (33, 16, True)])
def test_append_split(B, N, fp8):
    from mla_latent_kv_attn_amd.ops import Cache
    inp = make_append_inputs(B, D, seed=100 + B)
    rng = np.random.default_rng(B)
    pos = rng.integers(0, N, size=B)
    pos[0] = N - 1
    if B > 1:
        pos[1] = 0
    lat0 = np.full((B, N, DC), SENT8 if fp8 else SENT16, dtype=np.uint8 if fp8 else np.uint16)
    rope0 = np.full((B, N, DR), SENT16, dtype=np.uint16)
    scale0 = np.full((B, N), SENTF, dtype=np.float32)
    lat = torch.from_numpy(lat0.copy()).cuda() if fp8 else _bf16_tensor(lat0)
    rope = _bf16_tensor(rope0)
    scale = torch.from_numpy(scale0.copy()).cuda() if fp8 else None
    _run(Cache.split(lat, rope, scale), inp, pos, B)
    ref = _oracle(inp, pos)
    lat_g = lat.cpu().numpy() if fp8 else _bits(lat)
    rope_g = _bits(rope)
    rows = (np.arange(B), pos)
    # untouched bytes
    mask = np.ones((B, N), bool)
    mask[rows] = False
    assert np.array_equal(lat_g[mask], lat0[mask]) and np.array_equal(rope_g[mask], rope0[mask])
    _check_bf16(rope_g[rows], ref["k_R"], "rope")
    if fp8:
        sc_g = scale.cpu().numpy()
        assert np.array_equal(sc_g[mask], scale0[mask])
        _check_fp8(lat_g[rows], sc_g[rows], ref["c"], ref["c_e4m3"], ref["c_scale"], "latent")
    else:
        _check_bf16(lat_g[rows], ref["c"], "latent")


def test_append_packed():
    from mla_latent_kv_attn_amd.ops import Cache
    B, N = 6, 100
    inp = make_append_inputs(B, D, seed=7)
    pos = np.array([99, 0, 31, 32, 50, 1])
    kv0 = np.full((B, N, DC + DR), SENT16, dtype=np.uint16)
    kv = _bf16_tensor(kv0)
    _run(Cache.packed(kv, DC), inp, pos, B)
    ref = _oracle(inp, pos)
    g = _bits(kv)
    rows = (np.arange(B), pos)
    mask = np.ones((B, N), bool)
    mask[rows] = False
    assert np.array_equal(g[mask], kv0[mask])
    _check_bf16(g[rows][:, :DC], ref["c"], "latent")
    _check_bf16(g[rows][:, DC:], ref["k_R"], "rope")


@pytest.mark.parametrize("fp8,B", [(False, 4), (True, 4), (False, 2), (False, 1)])
def test_append_paged(fp8, B):
    from mla_latent_kv_attn_amd.ops import Cache
    P, pages = 64, 6
    inp = make_append_inputs(B, D, seed=9)
    rng = np.random.default_rng(3)
    bt = rng.permutation(B * pages).astype(np.int32).reshape(B, pages)
    pos = np.array([6 * 64 - 1, 0, 63, 64])[:B]
    n_pool = B * pages
    if fp8:
        lat0 = np.full((n_pool, P, DC), SENT8, dtype=np.uint8)
        rope0 = np.full((n_pool, P, DR), SENT16, dtype=np.uint16)
        sc0 = np.full((n_pool, P), SENTF, dtype=np.float32)
        lat, rope, sc = torch.from_numpy(lat0.copy()).cuda(), _bf16_tensor(rope0), torch.from_numpy(sc0.copy()).cuda()
        cache = Cache(lat, rope, sc, torch.from_numpy(bt).cuda(), P)
    else:
        kv0 = np.full((n_pool, P, DC + DR), SENT16, dtype=np.uint16)
        kv = _bf16_tensor(kv0)
        cache = Cache.paged(kv, torch.from_numpy(bt).cuda(), DC)
    _run(cache, inp, pos, B)
    ref = _oracle(inp, pos)
    pg, sl = bt[np.arange(B), pos // P], pos % P
    mask = np.ones((n_pool, P), bool)
    mask[pg, sl] = False
    if fp8:
        lg, rg, sg = lat.cpu().numpy(), _bits(rope), sc.cpu().numpy()
        assert np.array_equal(lg[mask], lat0[mask]) and np.array_equal(rg[mask], rope0[mask])
        assert np.array_equal(sg[mask], sc0[mask])
        _check_fp8(lg[pg, sl], sg[pg, sl], ref["c"], ref["c_e4m3"], ref["c_scale"], "latent")
        _check_bf16(rg[pg, sl], ref["k_R"], "rope")
    else:
        g = _bits(kv)
        assert np.array_equal(g[mask], kv0[mask])
        _check_bf16(g[pg, sl][:, :DC], ref["c"], "latent")
        _check_bf16(g[pg, sl][:, DC:], ref["k_R"], "rope")


def test_append_zero_hidden_state_and_large_positions():
    """h = 0 gives a zero latent (scale 1, codes 0) and a zero rope key; position 32767 exercises
    large rotation angles."""
    from mla_latent_kv_attn_amd.ops import Cache
    B, N = 3, 32768
    inp = make_append_inputs(B, D, seed=5)
    inp.h[0] = 0
    pos = np.array([5, 32767, 20000])
    lat = _bf16_tensor(np.full((B, N, DC), SENT16, dtype=np.uint16))
    rope = _bf16_tensor(np.full((B, N, DR), SENT16, dtype=np.uint16))
    _run(Cache.split(lat, rope), inp, pos, B)
    ref = _oracle(inp, pos)
    rows = (np.arange(B), pos)
    lg, rg = _bits(lat)[rows], _bits(rope)[rows]
    # zero values (the rotation may produce -0.0, which is the same value)
    assert np.all(decode_bf16(lg[0]) == 0) and np.all(decode_bf16(rg[0]) == 0)
    _check_bf16(lg, ref["c"], "latent")
    _check_bf16(rg, ref["k_R"], "rope")
    lat8 = torch.full((B, N, DC), SENT8, dtype=torch.uint8, device="cuda")
    sc = torch.full((B, N), SENTF, dtype=torch.float32, device="cuda")
    _run(Cache.split(lat8, rope, sc), inp, pos, B)
    assert float(sc[0, 5]) == 1.0 and int(lat8[0, 5].abs().sum()) == 0


@pytest.mark.parametrize("B,Dm", [(6, 1024), (3, 1024), (8, 2048)])
def test_append_short_rows(B, Dm):
    """A model width below 4096 at 5-8 tokens takes the two-pass form (the one-pass form is kept for
    the projection GEMV, which needs no workspace); at 3 tokens the GEMV serves the short rows."""
    from mla_latent_kv_attn_amd.ops import Cache
    N = 40
    inp = make_append_inputs(B, Dm, seed=200 + B)
    pos = (np.arange(B) * 7) % N
    lat0 = np.full((B, N, DC), SENT16, dtype=np.uint16)
    rope0 = np.full((B, N, DR), SENT16, dtype=np.uint16)
    lat, rope = _bf16_tensor(lat0), _bf16_tensor(rope0)
    _run(Cache.split(lat, rope), inp, pos, B)
    ref = _oracle(inp, pos)
    lat_g, rope_g = _bits(lat), _bits(rope)
    rows = (np.arange(B), pos)
    mask = np.ones((B, N), bool)
    mask[rows] = False
    assert np.array_equal(lat_g[mask], lat0[mask]) and np.array_equal(rope_g[mask], rope0[mask])
    _check_bf16(lat_g[rows], ref["c"], "latent")
    _check_bf16(rope_g[rows], ref["k_R"], "rope")
