"""One full absorbed decode step over preallocated buffers, all on one stream, through
mla_decode_step: for one bf16 sequence at the V3 head sizes (up to 4096 cached tokens) a single
kernel launch; otherwise mla_absorb_q -> mla_decode_partial_warm -> mla_decode_combine_uv (three
or four launches).  Buffers are allocated once (torch device memory) and reused, so a step is
nothing but those launches and can be captured in a HIP graph."""
from __future__ import annotations

import math

import torch

from . import ops


class DecodeStep:
    def __init__(self, B: int, H: int, d_h: int, d_c: int, d_R: int, max_len: int, q_dtype: torch.dtype,
                 device="cuda", num_splits: int = 0):
        self.B, self.H, self.d_h, self.d_c, self.d_R, self.max_len = B, H, d_h, d_c, d_R, max_len
        self.num_splits = num_splits
        self.scale = 1.0 / math.sqrt(d_h + d_R)
        self.q_abs = torch.empty((B, H, d_c), dtype=q_dtype, device=device)
        self.o_latent = torch.empty((B, H, d_c), dtype=torch.float32, device=device)
        self.lse = torch.empty((B, H), dtype=torch.float32, device=device)
        self.out = torch.empty((B, H, d_h), dtype=torch.float32, device=device)
        if num_splits:
            # an explicit split count: the three calls (the one-launch form has its own partition)
            nbytes = ops.mla_decode_workspace_bytes(B, H, d_c, max_len, num_splits)
            self.workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)
        else:
            self.workspace = ops.mla_decode_step_workspace(B, H, d_c, max_len, device)

    def __call__(self, q_C, q_R, W_UK, W_UV, cache: "ops.Cache", seq_lens, stream=None):
        if not self.num_splits:
            return ops.mla_decode_step(q_C, q_R, W_UK, W_UV, cache, seq_lens, self.max_len, self.workspace,
                                       out=self.out, q_abs=self.q_abs, o_latent=self.o_latent, lse=self.lse,
                                       scale=self.scale, stream=stream)
        ops.mla_absorb_q(q_C, W_UK, out=self.q_abs, stream=stream)
        # the partial pass warms W_UV into the cache with its spare workgroups (small batches)
        ops.mla_decode_partial_warm(self.q_abs, q_R, cache, seq_lens, self.max_len, self.scale, self.workspace,
                                    W_UV, num_splits=self.num_splits, stream=stream)
        ops.mla_decode_combine_uv(seq_lens, self.max_len, self.workspace, W_UV, self.o_latent, out=self.out,
                                  lse=self.lse, num_splits=self.num_splits, stream=stream)
        return self.out
