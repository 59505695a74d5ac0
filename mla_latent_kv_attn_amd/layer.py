"""One attention layer's decode step for one new token per sequence, every step in the library,
all on one stream over preallocated buffers (so the whole layer can be captured in a HIP graph):

  mla_cache_append   c = W_DKV h and k_R = RoPE_pos(W_KR h) written into the cache at row pos
  mla_query_proj     c_q = W_DQ h, q_C = W_UQ c_q, q_R = RoPE_pos(W_QR c_q)
  DecodeStep         q' = W_UK^T q_C, attention over the latent cache (rows < seq_lens), W_UV
  mla_out_proj       y = W_O o

For a bf16 cache the first two are one call, mla_query_proj_append: W_DQ, W_DKV and W_KR all
project h, so one pass over their stacked rows writes c_q and the new cache row together.

seq_lens[b] is normally pos[b] + 1: the new token attends to itself and everything before it.
"""
from __future__ import annotations

import torch

from . import ops
from .step import DecodeStep

WEIGHT_NAMES = ("W_DQ", "W_UQ", "W_QR", "W_DKV", "W_KR", "W_UK", "W_UV", "W_O")


class DecodeLayer:
    """weights: dict of bf16 device tensors W_DQ [d_q, D], W_UQ [H d_h, d_q], W_QR [H d_R, d_q],
    W_DKV [d_c, D], W_KR [d_R, D], W_UK / W_UV [H, d_h, d_c], W_O [D, H d_h]."""

    def __init__(self, weights: dict, cache: "ops.Cache", B: int, max_len: int, num_splits: int = 0,
                 rope_base: float = 10000.0, device="cuda"):
        missing = [k for k in WEIGHT_NAMES if k not in weights]
        if missing:
            raise ValueError(f"missing weights: {missing}")
        self.w, self.cache, self.B, self.max_len, self.rope_base = weights, cache, B, max_len, rope_base
        H, d_h, d_c = weights["W_UK"].shape
        d_q, D = weights["W_DQ"].shape
        d_R = weights["W_KR"].shape[0]
        self.H, self.D = H, D
        bf16 = torch.bfloat16
        self.c_q = torch.empty(B, d_q, dtype=bf16, device=device)
        self.q_C = torch.empty(B, H, d_h, dtype=bf16, device=device)
        self.q_R = torch.empty(B, H, d_R, dtype=bf16, device=device)
        self.y = torch.empty(B, D, dtype=torch.float32, device=device)

        def ws(n):
            return torch.empty(max(n, 16), dtype=torch.uint8, device=device)

        self.fused = cache.latent.dtype == torch.bfloat16 and cache.rope.dtype == torch.bfloat16
        self.append_ws = ws(ops.mla_cache_append_workspace_bytes(B, D))
        self.query_ws = ws(ops.mla_query_append_workspace_bytes(B, D, d_q, H, d_h, d_R, d_c) if self.fused
                           else ops.mla_query_workspace_bytes(B, D, d_q, H, d_h, d_R))
        self.out_ws = ws(ops.mla_proj_workspace_bytes(B, D, H * d_h))
        self.attn = DecodeStep(B, H, d_h, d_c, d_R, max_len, bf16, device=device, num_splits=num_splits)

    def __call__(self, h: torch.Tensor, pos: torch.Tensor, seq_lens: torch.Tensor, stream=None) -> torch.Tensor:
        w = self.w
        if self.fused:
            ops.mla_query_proj_append(h, w["W_DQ"], w["W_UQ"], w["W_QR"], w["W_DKV"], w["W_KR"], pos, self.cache,
                                      self.H, rope_base=self.rope_base, c_q=self.c_q, q_C=self.q_C, q_R=self.q_R,
                                      workspace=self.query_ws, stream=stream)
        else:
            ops.mla_cache_append(h, w["W_DKV"], w["W_KR"], pos, self.cache, rope_base=self.rope_base,
                                 workspace=self.append_ws, stream=stream)
            ops.mla_query_proj(h, w["W_DQ"], w["W_UQ"], w["W_QR"], pos, self.H, rope_base=self.rope_base,
                               c_q=self.c_q, q_C=self.q_C, q_R=self.q_R, workspace=self.query_ws, stream=stream)
        o = self.attn(self.q_C, self.q_R, w["W_UK"], w["W_UV"], self.cache, seq_lens, stream=stream)
        return ops.mla_out_proj(o, w["W_O"], out=self.y, workspace=self.out_ws, stream=stream)
