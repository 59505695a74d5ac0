"""Pins of the output-projection oracle (oracle/output.py): basis vectors, a hand-computed fold,
and the folded product of the latent outputs against W_O applied to the outputs of the
explicit-value decode oracle (already pinned by the worked example and closed forms).

A plausible slip fails one of them: W_O transposed or heads concatenated in another order
(basis vectors), W_UV folded transposed or on the wrong side (hand example, decode identity).
"""
import numpy as np
import pytest

import oracle
import oracle.output as oo
from tests._helpers import custom_inputs

PIN_CHECKS = []


def pin(fn):
    PIN_CHECKS.append(fn)
    return fn


@pin
def test_out_proj_basis_vectors():
    D, H, d_h = 5, 3, 2
    W_O = np.arange(D * H * d_h, dtype=np.float64).reshape(D, H * d_h) - 7.0
    for h, i in [(0, 0), (1, 1), (2, 0)]:
        o = np.zeros((1, H, d_h))
        o[0, h, i] = 1.0
        assert np.array_equal(oo.out_proj(W_O, o)[0], W_O[:, h * d_h + i])


@pin
def test_fold_hand_example():
    # D = 1, one head, d_h = 2, d_c = 1: W_O = [1 2], W_UV_h = [3; 4] -> W_OV = [11]
    W_O = np.array([[1.0, 2.0]])
    W_UV = np.array([[[3.0], [4.0]]])
    W_OV = oo.fold_o(W_O, W_UV)
    assert np.array_equal(W_OV, [[11.0]])
    assert np.array_equal(oo.out_proj_folded(W_OV, np.array([[[2.0]]])), [[22.0]])
    # D = 2, two heads, d_h = 1, d_c = 2: head h's block is W_O[:, h] W_UV_h
    W_O = np.array([[1.0, 2.0], [3.0, 4.0]])
    W_UV = np.array([[[5.0, 6.0]], [[7.0, 8.0]]])
    want = np.array([[5.0, 6.0, 14.0, 16.0], [15.0, 18.0, 28.0, 32.0]])
    assert np.array_equal(oo.fold_o(W_O, W_UV), want)


@pin
def test_folded_output_equals_w_o_of_explicit_value_decode():
    rng = np.random.default_rng(6)
    B, H, d_h, d_c, d_R, D = 2, 3, 4, 6, 2, 5
    lens = [5, 3]
    inp = custom_inputs(rng.standard_normal((B, H, d_h)), rng.standard_normal((B, H, d_R)),
                        rng.standard_normal((H, d_h, d_c)) * 0.5, rng.standard_normal((H, d_h, d_c)) * 0.5,
                        [rng.standard_normal((L, d_c)) for L in lens],
                        [rng.standard_normal((L, d_R)) for L in lens])
    ref = oracle.decode(inp)
    W_O = rng.standard_normal((D, H * d_h))
    y_explicit = oo.out_proj(W_O, ref["o"])                      # values expanded per token
    y_folded = oo.out_proj_folded(oo.fold_o(W_O, inp.W_UV), ref["o_lat"])
    assert np.allclose(y_folded, y_explicit, atol=1e-12, rtol=1e-12)


def _mut_out_proj_heads_minor(W_O, o):
    o = np.asarray(o, dtype=np.float64)
    return o.transpose(0, 2, 1).reshape(o.shape[0], -1) @ np.asarray(W_O, dtype=np.float64).T


def _mut_fold_uv_transposed(W_O, W_UV):
    W_UV = np.asarray(W_UV, dtype=np.float64)
    H, d_h, d_c = W_UV.shape
    return _ORIG_FOLD(W_O, W_UV.reshape(H, d_c, d_h).transpose(0, 2, 1))


def _mut_fold_heads_swapped(W_O, W_UV):
    return _ORIG_FOLD(W_O, np.asarray(W_UV)[::-1])


_ORIG_FOLD = oo.fold_o

MUTANTS = {
    "heads_minor_concat": ("out_proj", _mut_out_proj_heads_minor),
    "fold_reads_uv_transposed": ("fold_o", _mut_fold_uv_transposed),
    "fold_pairs_wrong_heads": ("fold_o", _mut_fold_heads_swapped),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistakes_are_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(oo, attr, fn)
    failures = 0
    for chk in PIN_CHECKS:
        try:
            chk()
        except (AssertionError, ValueError):
            failures += 1
    assert failures >= 1, f"planted mistake {name!r} passed every pin"
