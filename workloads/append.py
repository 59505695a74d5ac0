"""Seeded inputs of the cache-write step (hidden states and the two projections).

Draws (numpy PCG64, one SeedSequence spawned into [h, W_DKV, W_KR]):
  * h      ~ N(0, 1)       [B, D]   hidden states of the new tokens;
  * W_DKV  ~ N(0, 1/D)     [d_c, D] so that the latent components are ~N(0, 1);
  * W_KR   ~ N(0, 1/D)     [d_R, D].
All three are stored as bfloat16 bit patterns (nearest, ties to even).  The V3 hidden size is
D = 7168.  Nothing here computes the cache write itself.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from .gen import f32_to_bf16_bits


@dataclass
class AppendInputs:
    h: np.ndarray        # uint16 bf16 bits [B, D]
    W_DKV: np.ndarray    # uint16 bf16 bits [d_c, D]
    W_KR: np.ndarray     # uint16 bf16 bits [d_R, D]


def make_append_inputs(B: int, D: int = 7168, d_c: int = 512, d_R: int = 64, seed: int = 11) -> AppendInputs:
    s_h, s_dkv, s_kr = np.random.SeedSequence(seed).spawn(3)
    std = np.float32(1.0 / np.sqrt(D))
    h = np.random.Generator(np.random.PCG64(s_h)).standard_normal((B, D), dtype=np.float32)
    Wd = np.random.Generator(np.random.PCG64(s_dkv)).standard_normal((d_c, D), dtype=np.float32) * std
    Wr = np.random.Generator(np.random.PCG64(s_kr)).standard_normal((d_R, D), dtype=np.float32) * std
    return AppendInputs(h=f32_to_bf16_bits(h), W_DKV=f32_to_bf16_bits(Wd), W_KR=f32_to_bf16_bits(Wr))
