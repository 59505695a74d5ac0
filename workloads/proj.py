"""Seeded inputs of the projections around the attention core (query side and output side).

Query side (one SeedSequence spawned into [h, W_DQ, W_UQ, W_QR, W_UK, pos]):
  * h     ~ N(0, 1)          [B, D]        hidden states of the new tokens (V3: D = 7168);
  * W_DQ  ~ N(0, 1/D)        [d_q, D]      so that c_q is ~N(0, 1) (V3: d_q = 1536);
  * W_UQ  ~ N(0, 1/d_q)      [H d_h, d_q]  so that q_C is ~N(0, 1);
  * W_QR  ~ N(0, 1/d_q)      [H d_R, d_q];
  * W_UK  ~ N(0, 1/d_h)      [H, d_h, d_c] so that q' is ~N(0, 1);
  * pos   uniform integers in [0, max_pos)  [B]  positions of the new tokens.
Folded query (one SeedSequence spawned into [c_q, W_QK]):
  * c_q   ~ N(0, 1)          [B, d_q]      compressed queries;
  * W_QK  ~ N(0, 1/d_q)      [H, d_c, d_q] a folded absorbed query projection.
Output side (one SeedSequence spawned into [o, o_lat, W_O, W_UV]):
  * o     ~ N(0, 1)          [B, H, d_h]   float32 head outputs;
  * o_lat ~ N(0, 1)          [B, H, d_c]   float32 latent outputs;
  * W_O   ~ N(0, 1/(H d_h))  [D, H d_h];
  * W_UV  ~ N(0, 1/d_c)      [H, d_h, d_c].
Weights and h are stored as bfloat16 bit patterns (nearest, ties to even).  Nothing here computes
a projection.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from .gen import f32_to_bf16_bits


def _normal(seq, shape, std):
    g = np.random.Generator(np.random.PCG64(seq))
    x = g.standard_normal(shape, dtype=np.float32)
    return x * np.float32(std)


@dataclass
class QueryInputs:
    h: np.ndarray        # uint16 bf16 bits [B, D]
    W_DQ: np.ndarray     # uint16 [d_q, D]
    W_UQ: np.ndarray     # uint16 [H d_h, d_q]
    W_QR: np.ndarray     # uint16 [H d_R, d_q]
    W_UK: np.ndarray     # uint16 [H, d_h, d_c]
    pos: np.ndarray      # int32 [B]


def make_query_inputs(B: int, D: int = 7168, d_q: int = 1536, H: int = 128, d_h: int = 128, d_R: int = 64,
                      d_c: int = 512, seed: int = 21, max_pos: int = 32768) -> QueryInputs:
    s = np.random.SeedSequence(seed).spawn(6)
    pos = np.random.Generator(np.random.PCG64(s[5])).integers(0, max_pos, size=B).astype(np.int32)
    return QueryInputs(
        h=f32_to_bf16_bits(_normal(s[0], (B, D), 1.0)),
        W_DQ=f32_to_bf16_bits(_normal(s[1], (d_q, D), 1.0 / np.sqrt(D))),
        W_UQ=f32_to_bf16_bits(_normal(s[2], (H * d_h, d_q), 1.0 / np.sqrt(d_q))),
        W_QR=f32_to_bf16_bits(_normal(s[3], (H * d_R, d_q), 1.0 / np.sqrt(d_q))),
        W_UK=f32_to_bf16_bits(_normal(s[4], (H, d_h, d_c), 1.0 / np.sqrt(d_h))),
        pos=pos)


def make_folded_query_inputs(B: int, H: int = 128, d_c: int = 512, d_q: int = 1536, seed: int = 41):
    """(c_q [B, d_q], W_QK [H, d_c, d_q]) as bf16 bit patterns."""
    s = np.random.SeedSequence(seed).spawn(2)
    return (f32_to_bf16_bits(_normal(s[0], (B, d_q), 1.0)),
            f32_to_bf16_bits(_normal(s[1], (H, d_c, d_q), 1.0 / np.sqrt(d_q))))


@dataclass
class OutputInputs:
    o: np.ndarray        # float32 [B, H, d_h]
    o_lat: np.ndarray    # float32 [B, H, d_c]
    W_O: np.ndarray      # uint16 bf16 bits [D, H d_h]
    W_UV: np.ndarray     # uint16 [H, d_h, d_c]


def make_output_inputs(B: int, D: int = 7168, H: int = 128, d_h: int = 128, d_c: int = 512,
                       seed: int = 31) -> OutputInputs:
    s = np.random.SeedSequence(seed).spawn(4)
    return OutputInputs(
        o=_normal(s[0], (B, H, d_h), 1.0),
        o_lat=_normal(s[1], (B, H, d_c), 1.0),
        W_O=f32_to_bf16_bits(_normal(s[2], (D, H * d_h), 1.0 / np.sqrt(H * d_h))),
        W_UV=f32_to_bf16_bits(_normal(s[3], (H, d_h, d_c), 1.0 / np.sqrt(d_c))))
