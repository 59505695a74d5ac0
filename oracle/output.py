"""Plain CPU reference of the output projection of one decode step (test infrastructure only).

Followed step by step (cited by page title and section):

* The heads' outputs o_h = W_UV_h (sum_j a_j c_j) are concatenated and multiplied by the output
  matrix W_O ("The Journey to Multi-Head Latent Attention", section "The absorption trick (the
  magic)": the attention output of a token is the value sum followed by W_O).
* Because W_UV and W_O are both fixed, they can be folded once into one matrix per head,
  W_OV_h = W_O[:, h] W_UV_h, that maps the latent value sum of head h straight to the output
  ("Grouped-query and latent attention", section "The absorption trick": W_UV can be merged into
  W_O; "The Journey ...", same section).

Readings where the pages leave a step open (listed in the design doc):
* W_O is [D, H d_h], head h owning columns h d_h .. (h+1) d_h - 1 (the concatenation order of
  the heads); W_UV is [H, d_h, d_c] (v_C = W_UV_h c), the decode path's layout.
* The folded matrix is stored [D, H d_c], head h owning columns h d_c .. (h+1) d_c - 1, so the
  folded product reads the latent outputs [B, H, d_c] as one [B, H d_c] row per token.

Arithmetic is float64.  Parity status: every function here is pinned in
tests/test_oracle_output.py (basis vectors, a hand-computed fold, and the folded product of the
latent outputs against W_O applied to the outputs of the explicit-value decode).
"""
from __future__ import annotations

import numpy as np


def out_proj(W_O, o) -> np.ndarray:
    """y = W_O concat_h(o_h): W_O [D, H d_h], o [B, H, d_h] -> [B, D]."""
    W_O = np.asarray(W_O, dtype=np.float64)
    o = np.asarray(o, dtype=np.float64)
    return o.reshape(o.shape[0], -1) @ W_O.T


def fold_o(W_O, W_UV) -> np.ndarray:
    """W_OV[:, h d_c:(h+1) d_c] = W_O[:, h d_h:(h+1) d_h] W_UV_h: -> [D, H d_c]."""
    W_O = np.asarray(W_O, dtype=np.float64)
    W_UV = np.asarray(W_UV, dtype=np.float64)
    H, d_h, _ = W_UV.shape
    return np.concatenate([W_O[:, h * d_h:(h + 1) * d_h] @ W_UV[h] for h in range(H)], axis=1)


def out_proj_folded(W_OV, o_lat) -> np.ndarray:
    """y = sum_h W_OV_h o_lat_h: W_OV [D, H d_c], o_lat [B, H, d_c] -> [B, D]."""
    W_OV = np.asarray(W_OV, dtype=np.float64)
    o_lat = np.asarray(o_lat, dtype=np.float64)
    return o_lat.reshape(o_lat.shape[0], -1) @ W_OV.T
