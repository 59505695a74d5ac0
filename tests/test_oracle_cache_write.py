"""Pins of the cache-write oracle (oracle/cache_write.py) against closed forms and invariants.

Each test fixes a value or property that a plausible slip would break: a transposed weight
(basis vectors), a wrong pairing or frequency in RoPE (single components, relative-position
property), a wrong rounding rule (bf16 / E4M3 ties), a wrong scale rule.
"""
import math

import numpy as np
import pytest

from oracle import decode_bf16, decode_e4m3
from oracle.cache_write import cache_row, encode_bf16, encode_e4m3, project, quantize_e4m3, rope


# ----------------------------------------------------------------------------- projection
def test_project_hand_example_and_basis():
    W = np.array([[1.0, 2.0, 3.0], [4.0, 5.0, 6.0]])        # d_out = 2, D = 3
    assert np.array_equal(project(W, np.array([[1.0, 0.0, -1.0]])), [[-2.0, -2.0]])
    # basis vector e_i selects column i of W (a transposed W would select a row)
    for i in range(3):
        e = np.zeros((1, 3))
        e[0, i] = 1.0
        assert np.array_equal(project(W, e)[0], W[:, i])


# ----------------------------------------------------------------------------- RoPE
def test_rope_position_zero_is_identity():
    x = np.random.default_rng(0).standard_normal((3, 64))
    assert np.allclose(rope(x, [0, 0, 0]), x, atol=0, rtol=0)


@pytest.mark.parametrize("p", [1, 7, 1000, 32767])
def test_rope_single_components(p):
    d, base = 64, 10000.0
    for i in [0, 1, 5, 31]:
        th = p * base ** (-2.0 * i / d)
        e = np.zeros((1, d))
        e[0, 2 * i] = 1.0                       # even component of pair i -> (cos, sin)
        y = rope(e, [p])[0]
        # (angles up to 32767 rad: the last bits of the angle differ between the two evaluations)
        assert y[2 * i] == pytest.approx(math.cos(th), abs=1e-10)
        assert y[2 * i + 1] == pytest.approx(math.sin(th), abs=1e-10)
        assert np.count_nonzero(np.abs(y) > 1e-15) <= 2
        e[0, 2 * i], e[0, 2 * i + 1] = 0.0, 1.0    # odd component -> (-sin, cos)
        y = rope(e, [p])[0]
        assert y[2 * i] == pytest.approx(-math.sin(th), abs=1e-10)
        assert y[2 * i + 1] == pytest.approx(math.cos(th), abs=1e-10)


def test_rope_two_dims_is_plain_rotation_by_position():
    y = rope(np.array([[1.0, 0.0]]), [2])[0]     # pair 0 turns by the position itself
    assert y == pytest.approx([math.cos(2.0), math.sin(2.0)], abs=1e-15)


def test_rope_invariants():
    rng = np.random.default_rng(1)
    q = rng.standard_normal((1, 64))
    k = rng.standard_normal((1, 64))
    # pair norms are kept
    y = rope(q, [123])
    assert np.allclose(np.hypot(y[:, 0::2], y[:, 1::2]), np.hypot(q[:, 0::2], q[:, 1::2]), rtol=1e-12)
    # rotations compose
    assert np.allclose(rope(rope(q, [40]), [2]), rope(q, [42]), atol=1e-12)
    # scores depend only on the position difference
    for m, n in [(5, 3), (100, 98), (2, 0), (77, 75)]:
        s = float((rope(q, [m]) @ rope(k, [n]).T)[0, 0])
        assert s == pytest.approx(float((rope(q, [2]) @ k.T)[0, 0]), abs=1e-10)


# ----------------------------------------------------------------------------- bf16
def test_encode_bf16_patterns_and_ties():
    cases = {1.0: 0x3F80, -2.5: 0xC020, 0.0: 0x0000,
             1.0 + 2.0 ** -8: 0x3F80,                 # tie -> even (1.0)
             1.0 + 3 * 2.0 ** -8: 0x3F82,             # tie -> even (1 + 2^-6)
             1.0 + 2.0 ** -8 + 2.0 ** -20: 0x3F81,    # just above the tie -> up
             2.0 ** -133: 0x0001,                     # smallest subnormal
             -(2.0 ** -126): 0x8080}                  # smallest normal, negative
    for x, bits in cases.items():
        assert int(encode_bf16(np.array([x]))[0]) == bits, x


def test_encode_bf16_round_trips_every_finite_pattern():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    exp = (bits.astype(np.uint32) >> 7) & 0xFF
    finite = bits[exp != 0xFF]
    finite = finite[finite != 0x8000]                 # -0 encodes as +0 (no sign of zero kept)
    assert np.array_equal(encode_bf16(decode_bf16(finite)), finite)


# ----------------------------------------------------------------------------- E4M3
def test_encode_e4m3_patterns_ties_and_clamp():
    cases = {448.0: 0x7E, 1000.0: 0x7E, -1000.0: 0xFE, 0.5: 0x30, 1.0: 0x38, -1.0: 0xB8,
             2.0 ** -9: 0x01,                  # smallest subnormal
             2.0 ** -10: 0x00,                 # tie between 0 and 2^-9 -> even (0)
             3 * 2.0 ** -10: 0x02,             # tie between codes 1 and 2 -> even (2)
             1.0625: 0x38,                     # tie between 1.0 (0x38) and 1.125 (0x39) -> 0x38
             1.1875: 0x3A,                     # tie between 1.125 and 1.25 (0x3A) -> 0x3A
             0.9375 * 2.0 ** -6: 0x08}         # tie between largest subnormal and 2^-6 -> 0x08
    for y, code in cases.items():
        assert int(encode_e4m3(np.array([y]))[0]) == code, y


def test_encode_e4m3_round_trips_every_finite_code():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F and c != 0x80], dtype=np.uint8)
    assert np.array_equal(encode_e4m3(decode_e4m3(codes)), codes)


def test_quantize_scale_rule():
    c = np.array([[0.0] * 8, [7.0, -7.0, 3.5, 0.0, 1e-3, -2.0, 6.9, 0.1]])
    codes, s = quantize_e4m3(c)
    assert s[0] == 1.0 and np.all(codes[0] == 0)          # all-zero latent: scale 1
    assert s[1] == np.float32(7.0 / 448.0)                  # amax / 448
    assert codes[1][0] == 0x7E and codes[1][1] == 0xFE      # the largest element maps to +-448
    deq = decode_e4m3(codes, s)
    # every element within half a spacing of the E4M3 grid (relative 2^-4, or 2^-10 absolute * s)
    err = np.abs(deq[1] - c[1])
    assert np.all(err <= np.maximum(np.abs(c[1]) * 2.0 ** -4, 2.0 ** -10 * float(s[1])) + 1e-12)


# ----------------------------------------------------------------------------- the row
def test_cache_row_storage_forms_are_consistent():
    rng = np.random.default_rng(2)
    B, D = 3, 96
    h = rng.standard_normal((B, D))
    Wd = rng.standard_normal((32, D)) / math.sqrt(D)
    Wr = rng.standard_normal((8, D)) / math.sqrt(D)
    pos = np.array([0, 5, 1000])
    r = cache_row(h, Wd, Wr, pos)
    assert np.allclose(r["k_R"][0], project(Wr, h)[0], atol=1e-12)        # position 0: unrotated
    for key, val in (("c_bf16", r["c"]), ("k_R_bf16", r["k_R"])):
        dec = decode_bf16(r[key])
        assert np.all(np.abs(dec - val) <= np.abs(val) * 2.0 ** -8 + 1e-40)
    raw = project(Wr, h)
    assert np.allclose(np.hypot(r["k_R"][:, 0::2], r["k_R"][:, 1::2]), np.hypot(raw[:, 0::2], raw[:, 1::2]))
