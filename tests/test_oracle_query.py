"""Pins of the query-side oracle (oracle/query.py) against hand values, closed forms, invariants
and the already-pinned explicit keys of the decode oracle.

Each pin is chosen so that a plausible slip fails it: a transposed weight (basis vectors), heads
sliced from the wrong rows (single-row weights), RoPE over the whole concatenated vector instead
of per head, or with another convention than the key's (single components, relative position),
a fold in the wrong order (hand example, explicit keys).
"""
import math

import numpy as np
import pytest

import oracle.query as oq
from oracle import expand_kv
from oracle.cache_write import rope

PIN_CHECKS = []


def pin(fn):
    PIN_CHECKS.append(fn)
    return fn


@pin
def test_q_down_basis_vectors():
    W = np.arange(12, dtype=np.float64).reshape(3, 4) - 5.0      # d_q = 3, D = 4
    for i in range(4):
        e = np.zeros((1, 4))
        e[0, i] = 1.0
        assert np.array_equal(oq.q_down(W, e)[0], W[:, i])


@pin
def test_q_up_head_slices():
    H, d_h, d_R, d_q = 3, 4, 2, 5
    for h, i in [(0, 0), (1, 3), (2, 1)]:
        W_UQ = np.zeros((H * d_h, d_q))
        W_UQ[h * d_h + i, 2] = 1.5
        W_QR = np.zeros((H * d_R, d_q))
        c_q = np.zeros((1, d_q))
        c_q[0, 2] = 2.0
        q_C, q_R = oq.q_up(W_UQ, W_QR, c_q, [0], H)
        want = np.zeros((1, H, d_h))
        want[0, h, i] = 3.0
        assert np.array_equal(q_C, want)
        assert np.array_equal(q_R, np.zeros((1, H, d_R)))


@pin
def test_q_r_rotates_each_head_separately():
    # head h, pair i of q_R turns by pos * 10000^(-2i/64), the same for every head
    H, d_R, d_q = 3, 64, 2
    p = 7
    for h, i in [(0, 0), (1, 3), (2, 31)]:
        W_QR = np.zeros((H * d_R, d_q))
        W_QR[h * d_R + 2 * i, 0] = 1.0                          # even component of pair i
        c_q = np.array([[1.0, 0.0]])
        _, q_R = oq.q_up(np.zeros((H * 4, d_q)), W_QR, c_q, [p], H)
        th = p * 10000.0 ** (-2.0 * i / 64)
        want = np.zeros((1, H, d_R))
        want[0, h, 2 * i] = math.cos(th)
        want[0, h, 2 * i + 1] = math.sin(th)
        assert np.allclose(q_R, want, atol=1e-14, rtol=0)


@pin
def test_q_r_position_zero_is_the_plain_projection():
    rng = np.random.default_rng(3)
    H, d_R, d_q = 4, 64, 24
    W_QR = rng.standard_normal((H * d_R, d_q))
    c_q = rng.standard_normal((2, d_q))
    _, q_R = oq.q_up(rng.standard_normal((H * 8, d_q)), W_QR, c_q, [0, 0], H)
    assert np.allclose(q_R.reshape(2, -1), c_q @ W_QR.T, atol=1e-13)


@pin
def test_rotary_score_depends_only_on_distance_to_the_key():
    # q_R at the new token's position m against a cache row's k_R rotated at its position n
    # (the cache write's rotation): the score is a function of m - n alone
    rng = np.random.default_rng(4)
    H, d_R, d_q = 2, 64, 16
    W_QR = rng.standard_normal((H * d_R, d_q))
    c_q = rng.standard_normal((1, d_q))
    k = rng.standard_normal((1, d_R))
    ref = None
    for m, n in [(9, 0), (10, 1), (500, 491), (12345, 12336)]:
        _, q_R = oq.q_up(np.zeros((H * 4, d_q)), W_QR, c_q, [m], H)
        s = q_R[0] @ rope(k, [n])[0]                      # [H]
        if ref is None:
            ref = s
        assert np.allclose(s, ref, atol=1e-9)
    # and not a constant: another distance changes it
    _, q_R = oq.q_up(np.zeros((H * 4, d_q)), W_QR, c_q, [20], H)
    assert not np.allclose(q_R[0] @ rope(k, [0])[0], ref, atol=1e-6)


@pin
def test_fold_hand_example():
    # one head, d_h = 1, d_c = 2, d_q = 1: W_UK_h = [1 2], W_UQ_h = [3]
    W_UK = np.array([[[1.0, 2.0]]])
    W_UQ = np.array([[3.0]])
    W_QK = oq.fold_q(W_UQ, W_UK)
    assert np.array_equal(W_QK, [[[3.0], [6.0]]])
    assert np.array_equal(oq.absorb_folded(W_QK, np.array([[2.0]])), [[[6.0, 12.0]]])
    # two heads, d_h = 2: W_QK_h = W_UK_h^T W_UQ_h worked by hand
    W_UK = np.array([[[1.0, 0.0, 2.0], [0.0, 1.0, 1.0]], [[0.0, 0.0, 1.0], [1.0, 0.0, 0.0]]])
    W_UQ = np.array([[1.0, 2.0], [3.0, 4.0], [5.0, 6.0], [7.0, 8.0]])
    want = np.array([[[1.0, 2.0], [3.0, 4.0], [5.0, 8.0]],
                     [[7.0, 8.0], [0.0, 0.0], [5.0, 6.0]]])
    assert np.array_equal(oq.fold_q(W_UQ, W_UK), want)


@pin
def test_folded_query_scores_equal_explicit_key_scores():
    # q'_h . c_j (folded, or absorbed after the up-projection) = q_C,h . (W_UK_h c_j), the
    # content term of the score against the explicit key built by expand_kv
    rng = np.random.default_rng(5)
    H, d_h, d_c, d_q, d_R, B, L = 3, 4, 6, 5, 2, 2, 7
    W_UQ = rng.standard_normal((H * d_h, d_q))
    W_QR = rng.standard_normal((H * d_R, d_q))
    W_UK = rng.standard_normal((H, d_h, d_c))
    c_q = rng.standard_normal((B, d_q))
    C = rng.standard_normal((L, d_c))
    q_C, _ = oq.q_up(W_UQ, W_QR, c_q, [0, 3], H)
    qf = oq.absorb_folded(oq.fold_q(W_UQ, W_UK), c_q)
    qa = oq.absorb(W_UK, q_C)
    for b in range(B):
        for h in range(H):
            K, _ = expand_kv(C, np.zeros((L, d_R)), W_UK[h], np.zeros((d_h, d_c)))
            explicit = K[:, :d_h] @ q_C[b, h]
            assert np.allclose(C @ qf[b, h], explicit, atol=1e-12)
            assert np.allclose(C @ qa[b, h], explicit, atol=1e-12)


def _mut_q_up_rope_whole_vector(W_UQ, W_QR, c_q, pos, H, base=10000.0):
    c_q = np.asarray(c_q, dtype=np.float64)
    B = c_q.shape[0]
    return (c_q @ np.asarray(W_UQ).T).reshape(B, H, -1), rope(c_q @ np.asarray(W_QR).T, pos, base).reshape(B, H, -1)


def _mut_q_up_head_major_transposed(W_UQ, W_QR, c_q, pos, H, base=10000.0):
    q_C, q_R = _ORIG_Q_UP(W_UQ, W_QR, c_q, pos, H, base)
    B, _, d_h = q_C.shape
    return q_C.reshape(B, d_h, H).transpose(0, 2, 1), q_R


def _mut_q_up_rotation_backwards(W_UQ, W_QR, c_q, pos, H, base=10000.0):
    return _ORIG_Q_UP(W_UQ, W_QR, c_q, -np.asarray(pos), H, base)


def _mut_fold_transposed_uk(W_UQ, W_UK):
    W_UK = np.asarray(W_UK, dtype=np.float64)
    H, d_h, d_c = W_UK.shape
    W2 = W_UK.reshape(H, d_c, d_h).transpose(0, 2, 1)
    return _ORIG_FOLD(W_UQ, W2)


_ORIG_Q_UP = oq.q_up
_ORIG_FOLD = oq.fold_q

MUTANTS = {
    "rope_over_all_heads": ("q_up", _mut_q_up_rope_whole_vector),
    "heads_interleaved": ("q_up", _mut_q_up_head_major_transposed),
    "rotation_sign": ("q_up", _mut_q_up_rotation_backwards),
    "fold_reads_uk_transposed": ("fold_q", _mut_fold_transposed_uk),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistakes_are_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(oq, attr, fn)
    failures = 0
    for chk in PIN_CHECKS:
        try:
            chk()
        except (AssertionError, ValueError):
            failures += 1
    assert failures >= 1, f"planted mistake {name!r} passed every pin"
