"""Small helpers shared by the tests (no attention arithmetic here)."""
from __future__ import annotations

import numpy as np

from workloads.configs import Workload
from workloads.gen import DecodeInputs


def custom_inputs(q_C, q_R, W_UK, W_UV, C_rows, R_rows, n_max=None) -> DecodeInputs:
    """Build an fp32 split-layout input record from explicit per-sequence rows.

    q_C [B,H,d_h], q_R [B,H,d_R], W_UK/W_UV [H,d_h,d_c], C_rows: list of [L_b, d_c],
    R_rows: list of [L_b, d_R].  Padding rows are NaN.
    """
    q_C = np.asarray(q_C, dtype=np.float32)
    q_R = np.asarray(q_R, dtype=np.float32)
    W_UK = np.asarray(W_UK, dtype=np.float32)
    W_UV = np.asarray(W_UV, dtype=np.float32)
    B, H, d_h = q_C.shape
    d_R = q_R.shape[2]
    d_c = W_UK.shape[2]
    lens = np.array([len(c) for c in C_rows], dtype=np.int32)
    N = int(n_max if n_max is not None else max(1, lens.max(initial=1)))
    wl = Workload("custom", seed=0, B=B, H=H, d_h=d_h, d_c=d_c, d_R=d_R, n_max=N,
                  len_lo=int(lens.min(initial=0)), len_hi=int(lens.max(initial=0)),
                  dtype="f32", layout="split")
    lat = np.full((B, N, d_c), np.nan, dtype=np.float32)
    rope = np.full((B, N, d_R), np.nan, dtype=np.float32)
    for b in range(B):
        L = lens[b]
        if L:
            lat[b, :L] = np.asarray(C_rows[b], dtype=np.float32)
            rope[b, :L] = np.asarray(R_rows[b], dtype=np.float32)
    return DecodeInputs(wl=wl, lens=lens, q_C=q_C, q_R=q_R, W_UK=W_UK, W_UV=W_UV,
                        latent=lat, rope=rope)
