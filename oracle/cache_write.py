"""Plain CPU reference of the cache write of one decode step (test infrastructure only).

What a new token adds to a layer's cache, followed step by step (cited by page title and
section):

* The joint down-projection of the token's hidden state gives the latent,
  c = W_DKV h ("Grouped-query and latent attention", section "Multi-head
  latent attention (MLA)", column-vector form; "MLA storage: Representing KV
  with a small latent vector", section "Forming head-specific K and V from a
  small vector", row-vector form c = x W^D).
* A separate projection followed by RoPE at the token's position gives the
  positional key shared by all heads, k_R = RoPE_pos(W_KR h) ("MLA storage
  ...", section "Storing a positional key separately"; "Grouped-query and
  latent attention", section "Why a separate rotary key").
* Both are appended as one new cache row at that position ("MLA storage ...",
  same section).

Readings where the pages leave a step open (listed in the design doc):
* RoPE pairs components (2i, 2i+1) and turns pair i by pos * base^(-2i/d_R),
  base 10000; positions are 0-based row indices.
* Storage: bfloat16 is round-to-nearest-even of the exact value; the fp8 form
  is OCP E4M3 with a per-token float32 scale s = amax / 448 over the latent
  (s = 1 when amax = 0) and codes RNE(clamp(c / s, -448, 448)).

The encoders below are written from the formats' definitions (the E4M3 value
table of mla_decode) and share nothing with the input generator or the GPU
kernels.  Arithmetic is float64.

Parity status: every function here is pinned by closed forms and invariants in
tests/test_oracle_cache_write.py (basis-vector projections, RoPE at position 0,
pair norms, angles of single components, the relative-position property,
composition of rotations, bf16 and E4M3 bit patterns including ties, the scale
rule).
"""
from __future__ import annotations

from typing import Tuple

import numpy as np

from .mla_decode import _E4M3_TABLE


# --------------------------------------------------------------------------
# projections and rotation
# --------------------------------------------------------------------------
def project(W, h) -> np.ndarray:
    """Column-vector projection y = W h for every token: W [d_out, D], h [B, D] -> [B, d_out]."""
    W = np.asarray(W, dtype=np.float64)
    h = np.asarray(h, dtype=np.float64)
    return h @ W.T


def rope(x, pos, base: float = 10000.0) -> np.ndarray:
    """Rotate each pair (x[2i], x[2i+1]) of every row by angle pos * base**(-2i/d).

    x [B, d] (d even), pos [B] integer positions.
    """
    x = np.asarray(x, dtype=np.float64)
    pos = np.asarray(pos, dtype=np.float64)
    d = x.shape[-1]
    i = np.arange(d // 2, dtype=np.float64)
    theta = pos[:, None] * base ** (-2.0 * i / d)[None, :]   # [B, d/2]
    c, s = np.cos(theta), np.sin(theta)
    even, odd = x[:, 0::2], x[:, 1::2]
    out = np.empty_like(x)
    out[:, 0::2] = even * c - odd * s
    out[:, 1::2] = even * s + odd * c
    return out


# --------------------------------------------------------------------------
# storage encoding
# --------------------------------------------------------------------------
def encode_bf16(x) -> np.ndarray:
    """float64 -> bfloat16 bit patterns, round to nearest, ties to even (finite inputs).

    A bf16 number has 8 significant bits: for |x| in [2^e, 2^(e+1)) the spacing is 2^(e-7),
    and below 2^-126 (subnormal) it is 2^-133.
    """
    x = np.asarray(x, dtype=np.float64)
    ax = np.abs(x)
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(ax > 0, ax, 1.0)))
    e = np.maximum(e, -126.0)
    ulp = np.exp2(e - 7.0)
    v = np.rint(x / ulp) * ulp          # np.rint: round half to even
    v = np.where(ax > 0, v, x)
    if np.any(np.abs(v) > 3.3895313892515355e38):
        raise OverflowError("value outside the bfloat16 range")
    return (v.astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)


_POS_CODES = np.arange(0, 0x7F, dtype=np.int64)            # +0 .. +448 (0x7F is NaN)
_POS_VALUES = _E4M3_TABLE[_POS_CODES]                       # increasing


def encode_e4m3(y) -> np.ndarray:
    """float64 -> OCP E4M3 codes: clamp to [-448, 448], then the nearest value, ties to the even
    code (even mantissa bit).  -0.0 and values that round to zero encode as +0 / -0 by sign."""
    y = np.clip(np.asarray(y, dtype=np.float64), -448.0, 448.0)
    a = np.abs(y)
    hi = np.searchsorted(_POS_VALUES, a, side="left")        # first value >= a
    hi = np.minimum(hi, len(_POS_VALUES) - 1)
    lo = np.maximum(hi - 1, 0)
    dlo = a - _POS_VALUES[lo]
    dhi = _POS_VALUES[hi] - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (_POS_CODES[hi] % 2 == 0))
    code = np.where(pick_hi, _POS_CODES[hi], _POS_CODES[lo]).astype(np.uint8)
    return np.where(np.signbit(y) & (code != 0), code | np.uint8(0x80), code).astype(np.uint8)


def quantize_e4m3(c) -> Tuple[np.ndarray, np.ndarray]:
    """Per-row E4M3 codes and float32 scales of latents c [B, d_c]: s = amax / 448 (1 if amax = 0)."""
    c = np.asarray(c, dtype=np.float64)
    amax = np.max(np.abs(c), axis=-1)
    s = np.where(amax > 0, amax / 448.0, 1.0).astype(np.float32)
    codes = encode_e4m3(c / s.astype(np.float64)[:, None])
    return codes, s


# --------------------------------------------------------------------------
# the new cache row
# --------------------------------------------------------------------------
def cache_row(h, W_DKV, W_KR, pos, base: float = 10000.0) -> dict:
    """Exact (float64) latent and rotated rope key of the new token of every sequence, and their
    storage forms.  h [B, D], W_DKV [d_c, D], W_KR [d_R, D], pos [B]."""
    c = project(W_DKV, h)
    kr = rope(project(W_KR, h), pos, base)
    codes, scale = quantize_e4m3(c)
    return {"c": c, "k_R": kr, "c_bf16": encode_bf16(c), "k_R_bf16": encode_bf16(kr),
            "c_e4m3": codes, "c_scale": scale}
