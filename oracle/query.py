"""Plain CPU reference of the query side of one decode step (test infrastructure only).

Followed step by step (cited by page title and section):

* The new token's hidden state h is compressed to c_q = W_DQ h, and the per-head content
  queries are its up-projection q_C = W_UQ c_q ("Grouped-query and latent attention", section
  "Multi-head latent attention (MLA)": d_q = 1536 in DeepSeek-V3).
* The positional query of every head is q_R = RoPE(W_QR c_q), of dimension d_R = 64 per head
  (same page, section "Why a separate rotary key").
* The absorbed query of head h is q'_h = W_UK_h^T q_C,h (same page, section "The absorption
  trick"); because W_UQ and W_UK are both fixed, they can be folded once into one "absorbed
  query projection" W_QK_h = W_UK_h^T W_UQ_h, and then q'_h = W_QK_h c_q ("The Journey to
  Multi-Head Latent Attention", section "The absorption trick (the magic)").

Readings where the pages leave a step open (listed in the design doc):
* W_UQ is [H d_h, d_q] and W_QR is [H d_R, d_q], head h owning rows h d_h .. (h+1) d_h - 1
  (resp. h d_R ..); W_UK is [H, d_h, d_c] (k_C = W_UK_h c), the decode path's layout.
* The rotation of q_R is the one the cache write applies to k_R (pairs (2i, 2i+1) of each
  head's 64 components turned by pos * base^(-2i/64), base 10000) at the new token's position,
  so that a score's rotary term depends only on the distance between query and key.
* No normalisation sits between the projections: the pages name none.

Arithmetic is float64.  Parity status: every function here is pinned in
tests/test_oracle_query.py (basis vectors and head slices of the projections, single rotary
components per head, the relative-position property against the cache write's k_R, a
hand-computed fold, and the fold against explicit keys from expand_kv).
"""
from __future__ import annotations

import numpy as np

from .cache_write import project, rope


def q_down(W_DQ, h) -> np.ndarray:
    """c_q = W_DQ h for every token: W_DQ [d_q, D], h [B, D] -> [B, d_q]."""
    return project(W_DQ, h)


def q_up(W_UQ, W_QR, c_q, pos, H: int, base: float = 10000.0):
    """Per-head content and rotated positional queries of every token.

    W_UQ [H d_h, d_q], W_QR [H d_R, d_q], c_q [B, d_q], pos [B].
    Returns q_C [B, H, d_h] and q_R [B, H, d_R].
    """
    c_q = np.asarray(c_q, dtype=np.float64)
    B = c_q.shape[0]
    q_C = project(W_UQ, c_q).reshape(B, H, -1)
    raw = project(W_QR, c_q).reshape(B, H, -1)
    d_R = raw.shape[-1]
    pos = np.asarray(pos)
    # every head's d_R components rotate like the key's, at the token's position
    q_R = rope(raw.reshape(B * H, d_R), np.repeat(pos, H), base).reshape(B, H, d_R)
    return q_C, q_R


def absorb(W_UK, q_C) -> np.ndarray:
    """q'[b, h] = W_UK_h^T q_C[b, h]: W_UK [H, d_h, d_c], q_C [B, H, d_h] -> [B, H, d_c]."""
    W_UK = np.asarray(W_UK, dtype=np.float64)
    q_C = np.asarray(q_C, dtype=np.float64)
    return np.stack([q_C[:, h, :] @ W_UK[h] for h in range(W_UK.shape[0])], axis=1)


def fold_q(W_UQ, W_UK) -> np.ndarray:
    """Absorbed query projection W_QK_h = W_UK_h^T W_UQ_h: -> [H, d_c, d_q]."""
    W_UQ = np.asarray(W_UQ, dtype=np.float64)
    W_UK = np.asarray(W_UK, dtype=np.float64)
    H, d_h, _ = W_UK.shape
    return np.stack([W_UK[h].T @ W_UQ[h * d_h:(h + 1) * d_h] for h in range(H)])


def absorb_folded(W_QK, c_q) -> np.ndarray:
    """q'[b, h] = W_QK_h c_q[b]: W_QK [H, d_c, d_q], c_q [B, d_q] -> [B, H, d_c]."""
    W_QK = np.asarray(W_QK, dtype=np.float64)
    c_q = np.asarray(c_q, dtype=np.float64)
    return np.einsum("hkj,bj->bhk", W_QK, c_q)
