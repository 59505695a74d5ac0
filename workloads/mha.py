"""Seeded inputs of the same-dimension MHA comparison (explicit per-head K/V caches).

Draws (numpy PCG64, one SeedSequence spawned into [q, K, V]): q ~ N(0, 1) [B, H, 192],
K ~ N(0, 1) [B, H, cap, 192], V ~ N(0, 1) [B, H, cap, 128], stored as bfloat16 bit patterns;
rows at or past each sequence's length are filled with NaN (a kernel that reads them into the
result produces a non-finite output).  Nothing here computes attention.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from .gen import BF16_NAN, f32_to_bf16_bits


@dataclass
class MhaInputs:
    lens: np.ndarray   # int32 [B]
    q: np.ndarray      # uint16 [B, H, 192]
    K: np.ndarray      # uint16 [B, H, cap, 192]
    V: np.ndarray      # uint16 [B, H, cap, 128]


def make_mha_inputs(lens, H: int, cap: int, seed: int = 21, d_k: int = 192, d_v: int = 128) -> MhaInputs:
    lens = np.asarray(lens, dtype=np.int32)
    B = len(lens)
    s_q, s_k, s_v = np.random.SeedSequence(seed).spawn(3)
    q = np.random.Generator(np.random.PCG64(s_q)).standard_normal((B, H, d_k), dtype=np.float32)
    K = f32_to_bf16_bits(np.random.Generator(np.random.PCG64(s_k)).standard_normal((B, H, cap, d_k), dtype=np.float32))
    V = f32_to_bf16_bits(np.random.Generator(np.random.PCG64(s_v)).standard_normal((B, H, cap, d_v), dtype=np.float32))
    for b in range(B):
        K[b, :, lens[b]:] = BF16_NAN
        V[b, :, lens[b]:] = BF16_NAN
    return MhaInputs(lens=lens, q=f32_to_bf16_bits(q), K=K, V=V)
