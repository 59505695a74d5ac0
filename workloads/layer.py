"""Seeded inputs of one attention layer's decode step (one new token per sequence).

One SeedSequence spawned into [h, W_DQ, W_UQ, W_QR, W_DKV, W_KR, W_UK, W_UV, W_O, cache]:
  * h ~ N(0, 1) [B, D]; W_DQ, W_DKV, W_KR ~ N(0, 1/D); W_UQ, W_QR ~ N(0, 1/d_q);
    W_UK, W_UV ~ N(0, 1/d_c) [H, d_h, d_c] (as the decode workloads); W_O ~ N(0, 1/(H d_h));
  * the cache already holds lens[b] rows per sequence: latents ~ N(0, 1) and rope keys ~ N(0, 1)
    (stored values, as the decode workloads draw them); rows from lens[b] on are NaN, so a read
    past the sequence shows;
  * the new token of sequence b goes to row pos[b] = lens[b].
Everything is stored as bfloat16 bit patterns (nearest, ties to even), the split cache layout
[B, cap, 512] + [B, cap, 64].  Nothing here computes any step of the layer.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

from .gen import f32_to_bf16_bits

_NAN_BF16 = np.uint16(0x7FC0)


@dataclass
class LayerInputs:
    h: np.ndarray                  # uint16 [B, D]
    weights: dict = field(default_factory=dict)   # name -> uint16 array
    latent: np.ndarray = None      # uint16 [B, cap, d_c]
    rope: np.ndarray = None        # uint16 [B, cap, d_R]
    lens: np.ndarray = None        # int32 [B] rows already cached
    pos: np.ndarray = None         # int32 [B] row of the new token (= lens)


def make_layer_inputs(lens, cap: int, D: int = 7168, d_q: int = 1536, H: int = 128, d_h: int = 128,
                      d_c: int = 512, d_R: int = 64, seed: int = 51) -> LayerInputs:
    lens = np.asarray(lens, dtype=np.int32)
    B = len(lens)
    if np.any(lens >= cap):
        raise ValueError("every sequence needs a free row for the new token")
    s = np.random.SeedSequence(seed).spawn(10)

    def normal(i, shape, std):
        return np.random.Generator(np.random.PCG64(s[i])).standard_normal(shape, dtype=np.float32) * np.float32(std)

    shapes = {"W_DQ": ((d_q, D), 1 / np.sqrt(D)), "W_UQ": ((H * d_h, d_q), 1 / np.sqrt(d_q)),
              "W_QR": ((H * d_R, d_q), 1 / np.sqrt(d_q)), "W_DKV": ((d_c, D), 1 / np.sqrt(D)),
              "W_KR": ((d_R, D), 1 / np.sqrt(D)), "W_UK": ((H, d_h, d_c), 1 / np.sqrt(d_c)),
              "W_UV": ((H, d_h, d_c), 1 / np.sqrt(d_c)), "W_O": ((D, H * d_h), 1 / np.sqrt(H * d_h))}
    weights = {k: f32_to_bf16_bits(normal(i + 1, shp, std)) for i, (k, (shp, std)) in enumerate(shapes.items())}
    g = np.random.Generator(np.random.PCG64(s[9]))
    latent = np.full((B, cap, d_c), _NAN_BF16, dtype=np.uint16)
    rope = np.full((B, cap, d_R), _NAN_BF16, dtype=np.uint16)
    for b in range(B):
        L = int(lens[b])
        latent[b, :L] = f32_to_bf16_bits(g.standard_normal((L, d_c), dtype=np.float32))
        rope[b, :L] = f32_to_bf16_bits(g.standard_normal((L, d_R), dtype=np.float32))
    return LayerInputs(h=f32_to_bf16_bits(normal(0, (B, D), 1.0)), weights=weights, latent=latent, rope=rope,
                       lens=lens, pos=lens.copy())
