"""Input generator checks: determinism, storage encoders, rotary invariants, layouts."""
from __future__ import annotations

import math

import numpy as np
import pytest

import oracle
from workloads import make_inputs, WORKLOADS
from workloads.configs import Workload
from workloads.gen import (bf16_bits_to_f32, encode_e4m3, f32_to_bf16_bits, quantize_rows_e4m3,
                           rope_rotate)


def small(layout="split", dtype="bf16", **kw):
    base = dict(name="small", seed=11, B=3, H=4, d_h=16, d_c=64, d_R=8, n_max=192,
                len_lo=1, len_hi=192, dtype=dtype, layout=layout)
    base.update(kw)
    return Workload(**base)


def test_seed_determinism_and_lengths():
    a = make_inputs(small())
    b = make_inputs(small())
    c = make_inputs(small(), seed=12)
    np.testing.assert_array_equal(a.latent, b.latent)
    np.testing.assert_array_equal(a.q_R, b.q_R)
    assert not np.array_equal(a.W_UK, c.W_UK)
    assert a.lens.min() >= 1 and a.lens.max() <= 192
    # threading must not change the draws
    d = make_inputs(small(), threads=1)
    np.testing.assert_array_equal(a.latent, d.latent)


def test_padding_is_poisoned_and_valid_rows_finite():
    inp = make_inputs(small())
    for b in range(inp.wl.B):
        L = inp.lens[b]
        assert np.all(inp.latent[b, L:] == 0x7FC0)
        assert np.all(np.isfinite(bf16_bits_to_f32(inp.latent[b, :L])))


def test_bf16_round_to_nearest_even():
    x = np.array([1.0, 1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, 1 + 2.0 ** -8 + 2.0 ** -20, -2.5, 3.0e38, np.nan],
                 dtype=np.float32)
    r = f32_to_bf16_bits(x)
    assert r[0] == 0x3F80
    assert r[1] == 0x3F80          # tie -> even (mantissa 0)
    assert r[2] == 0x3F82          # tie -> even (mantissa 2)
    assert r[3] == 0x3F81          # above the tie -> up
    assert oracle.decode_bf16(r[4]) == -2.5
    assert r[6] == 0x7FC0
    rng = np.random.default_rng(0)
    y = rng.standard_normal(100000).astype(np.float32)
    back = bf16_bits_to_f32(f32_to_bf16_bits(y))
    assert np.max(np.abs(back - y) / np.abs(y)) <= 2.0 ** -8


def test_e4m3_encoder_roundtrips_every_finite_code():
    codes = np.arange(256, dtype=np.uint8)
    vals = oracle.decode_e4m3(codes)
    fin = np.isfinite(vals)
    enc = encode_e4m3(vals[fin].astype(np.float32))
    np.testing.assert_array_equal(enc, codes[fin])


def test_e4m3_encoder_rounds_to_nearest_even():
    # between 1.0 (0x38) and 1.125 (0x39): the midpoint goes to the even mantissa 0x38
    assert encode_e4m3(np.float32(1.0625)) == 0x38
    # between 1.125 (0x39) and 1.25 (0x3A): the midpoint goes to 0x3A
    assert encode_e4m3(np.float32(1.1875)) == 0x3A
    # subnormal midpoint between 2^-9 (0x01) and 2*2^-9 (0x02): to 0x02
    assert encode_e4m3(np.float32(1.5 * 2.0 ** -9)) == 0x02
    # just below the smallest normal rounds up into it
    assert encode_e4m3(np.float32(2.0 ** -6 - 2.0 ** -12)) == 0x08
    assert encode_e4m3(np.float32(448.0)) == 0x7E and encode_e4m3(np.float32(-448.0)) == 0xFE


def test_per_token_scaled_fp8_bounds():
    rng = np.random.default_rng(3)
    rows = rng.standard_normal((2000, 512)).astype(np.float32)
    rows[5] = 0.0
    codes, scale = quantize_rows_e4m3(rows)
    assert scale[5] == 1.0
    deq = oracle.decode_e4m3(codes, scale)
    assert np.all(np.isfinite(deq))
    amax = np.abs(rows).max(axis=1)
    np.testing.assert_allclose(np.abs(deq).max(axis=1), amax, rtol=2.0 ** -4)
    y = rows / scale[:, None]
    big = np.abs(y) >= 2.0 ** -6
    rel = np.abs(deq - rows)[big] / np.abs(rows)[big]
    assert rel.max() <= 2.0 ** -4 + 1e-7
    absd = np.abs(deq - rows)[~big] / np.broadcast_to(scale[:, None], rows.shape)[~big]
    assert absd.max() <= 2.0 ** -10 + 1e-12
    # every e4m3 value is exactly a bf16 value
    vals = oracle.decode_e4m3(np.arange(256, dtype=np.uint8))
    vals = vals[np.isfinite(vals)].astype(np.float32)
    assert np.array_equal(bf16_bits_to_f32(f32_to_bf16_bits(vals)), vals)


def test_rope_relative_position_and_norm():
    rng = np.random.default_rng(4)
    q = rng.standard_normal(64)
    k = rng.standard_normal(64)
    for m, n, shift in [(3, 10, 5), (0, 4095, 100), (17, 2, 1000)]:
        s1 = rope_rotate(q, m) @ rope_rotate(k, n)
        s2 = rope_rotate(q, m + shift) @ rope_rotate(k, n + shift)
        assert s1 == pytest.approx(s2, rel=1e-9, abs=1e-9)
        assert np.linalg.norm(rope_rotate(k, n)) == pytest.approx(np.linalg.norm(k), rel=1e-12)
    np.testing.assert_allclose(rope_rotate(k, 0), k, rtol=0, atol=0)


def test_rotation_on_expanded_key_breaks_the_fold():
    """Rotating the expanded key puts R(n-m) between q_C and W_UK, so the folded query
    would depend on the key position ("Grouped-query and latent attention", "Why a separate
    rotary key"): no single q' reproduces the scores of two positions."""
    rng = np.random.default_rng(5)
    d_h, d_c = 8, 12
    W = rng.standard_normal((d_h, d_c))
    q = rng.standard_normal(d_h)
    c = rng.standard_normal(d_c)
    folded = W.T @ q
    base = folded @ c
    assert q @ (W @ c) == pytest.approx(base, rel=1e-12)
    rotated = [rope_rotate(q, 7) @ rope_rotate(W @ c, n) for n in (0, 3, 11)]
    assert not all(r == pytest.approx(base, rel=1e-6) for r in rotated)


def test_paged_and_packed_hold_the_same_logical_rows():
    pk = make_inputs(small(layout="packed", n_max=256, len_hi=256))
    pg = make_inputs(small(layout="paged", n_max=256, len_hi=256, page_size=64))
    np.testing.assert_array_equal(pk.lens, pg.lens)
    bt = pg.block_table
    assert sorted(bt.reshape(-1).tolist()) == list(range(bt.size))
    for b in range(pk.wl.B):
        C1, R1 = oracle.gather_rows(pk, b)
        C2, R2 = oracle.gather_rows(pg, b)
        np.testing.assert_array_equal(C1, C2)
        np.testing.assert_array_equal(R1, R2)


def test_length_override_keeps_other_draws():
    a = make_inputs(small())
    lens = np.array([0, 1, 192], dtype=np.int32)
    b = make_inputs(small(), lens=lens)
    np.testing.assert_array_equal(a.W_UK, b.W_UK)
    np.testing.assert_array_equal(a.q_C, b.q_C)
    assert np.all(b.latent[0] == 0x7FC0)


def test_config_shapes():
    w = WORKLOADS
    assert (w[2].B, w[2].H, w[2].d_c, w[2].d_R, w[2].n_max) == (1, 128, 512, 64, 4096)
    assert w[3].layout == "packed" and w[4].layout == "paged" and w[5].dtype == "fp8"
    assert math.isclose(w[2].scale, 1 / math.sqrt(192)) and math.isclose(w[1].scale, 1 / math.sqrt(24))


def test_smoke_inputs_build_on_the_host():
    # the inputs of __graft_entry__.smoke() are built without a GPU
    import __graft_entry__ as g
    cases = g.smoke_inputs()
    assert len(cases) == 2
    assert list(cases[1][0].lens) == [96, 33, 1]
