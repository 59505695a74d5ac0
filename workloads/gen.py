"""Seeded input synthesis for the decode workloads.

What is drawn (all seeded, reproducible):
  * per-sequence lengths, uniform integers in [len_lo, len_hi];
  * W_UK, W_UV  ~ N(0, 1/d_c)               shape [H, d_h, d_c];
  * q_C, q_R    ~ N(0, 1)                    shape [B, H, d_h], [B, H, d_R];
  * latent rows ~ N(0, 1)                    shape [len_b, d_c] per sequence;
  * raw rope-key rows ~ N(0, 1)              shape [len_b, d_R] per sequence;
  * a permutation of physical pages for the paged layout.

The rope key and the rope query are stored *already rotated*: the cache-write
step of decoupled RoPE applies the rotation for the token's position before
the row is appended ("MLA storage: Representing KV with a small latent
vector", section "Storing a positional key separately"; "Grouped-query and
latent attention", section "Why a separate rotary key").  The pages do not fix
the pairing convention (the chapter on rotary embeddings that they refer to is
not part of the pages), so this generator rotates interleaved pairs
(2i, 2i+1) by pos * base**(-2i/d_R).  Key j sits at position j and the query
at position len_b - 1.

Storage formats:
  * "f32": float32 arrays;
  * "bf16": uint16 bit patterns, rounded once from float32 with
    round-to-nearest-even;
  * "fp8": OCP FP8 E4M3 ("e4m3fn": bias 7, max normal 448, no infinities,
    S.1111.111 is NaN) bit patterns with one float32 scale per token,
    scale = amax/448 over the token's latent components (scale 1 when the row
    is all zeros); the value is divided by the scale, clamped to +-448 and
    rounded to nearest even.  The rope key stays bf16.

Padding rows (j >= len_b) are filled with NaN when ``poison`` is true, so a
kernel that lets padding leak into the result produces a non-finite output.

Streams: a root ``numpy.random.SeedSequence(seed)`` is spawned into
[lengths, weights, queries, cache, pages]; the cache stream is spawned again
into one child per sequence, which draws that sequence's latent rows and then
its raw rope rows.  Sequences can therefore be generated independently.
"""
from __future__ import annotations

import concurrent.futures as _cf
import os
from dataclasses import dataclass, field
from typing import Optional

import numpy as np

from .configs import Workload, get_workload

BF16_NAN = np.uint16(0x7FC0)
E4M3_NAN = np.uint8(0x7F)
E4M3_MAX = 448.0


# --------------------------------------------------------------------------
# storage encoders
# --------------------------------------------------------------------------
def f32_to_bf16_bits(x) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        r[nan] = BF16_NAN
    return r


def bf16_bits_to_f32(b) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32 (generator-side helper)."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def encode_e4m3(y) -> np.ndarray:
    """Encode float32 values already clamped to [-448, 448] as OCP E4M3 bits (RNE).

    Normal codes hold (1 + m/8) * 2**(e-7) for e in 1..15; subnormal codes hold
    m * 2**-9.  NaN inputs map to 0x7F.
    """
    y = np.asarray(y, dtype=np.float32)
    a = np.abs(y).astype(np.float64)
    sign = (np.signbit(y)).astype(np.uint8) << 7
    code = np.zeros(y.shape, dtype=np.int32)
    sub = a < 2.0 ** -6
    # subnormal range: multiples of 2**-9; a count of 8 is the smallest normal (code 0x08)
    code[sub] = np.rint(a[sub] * 512.0).astype(np.int32)
    nrm = ~sub
    if nrm.any():
        mant, ex = np.frexp(a[nrm])          # a = mant * 2**ex, mant in [0.5, 1)
        e = ex - 1                           # a = (2*mant) * 2**e, 2*mant in [1, 2)
        m = np.rint((2.0 * mant - 1.0) * 8.0).astype(np.int32)
        carry = m == 8
        e = np.where(carry, e + 1, e)
        m = np.where(carry, 0, m)
        code[nrm] = ((e + 7) << 3) | m
    out = (code.astype(np.uint8) & 0x7F) | sign
    nan = np.isnan(y)
    if nan.any():
        out[nan] = E4M3_NAN
    return out.astype(np.uint8)


def quantize_rows_e4m3(rows: np.ndarray):
    """Per-row (per-token) scaled E4M3: scale = amax/448, code = e4m3(clamp(x/scale))."""
    rows = np.asarray(rows, dtype=np.float32)
    amax = np.max(np.abs(rows), axis=-1)
    scale = (amax / np.float32(E4M3_MAX)).astype(np.float32)
    scale = np.where(amax == 0, np.float32(1.0), scale).astype(np.float32)
    y = (rows / scale[..., None]).astype(np.float32)
    y = np.clip(y, -E4M3_MAX, E4M3_MAX).astype(np.float32)
    return encode_e4m3(y), scale


# --------------------------------------------------------------------------
# upstream cache-write step: rotary rotation of the rope key / query
# --------------------------------------------------------------------------
def rope_rotate(x: np.ndarray, pos, base: float = 10000.0) -> np.ndarray:
    """Rotate interleaved pairs (2i, 2i+1) of the last axis by pos * base**(-2i/d).

    ``pos`` broadcasts against x.shape[:-1].  Computed in float64.
    """
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    i = np.arange(d // 2, dtype=np.float64)
    inv = base ** (-2.0 * i / d)
    ang = np.asarray(pos, dtype=np.float64)[..., None] * inv
    c, s = np.cos(ang), np.sin(ang)
    x0, x1 = x[..., 0::2], x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = x0 * c - x1 * s
    out[..., 1::2] = x0 * s + x1 * c
    return out


# --------------------------------------------------------------------------
# the input record
# --------------------------------------------------------------------------
@dataclass
class DecodeInputs:
    """Host arrays for one decode step, in storage formats.

    bf16 tensors are uint16 bit patterns; fp8 latents are uint8 E4M3 codes.
    Cache arrays by layout:
      split : latent [B, n_max, d_c], rope [B, n_max, d_R], scale [B, n_max] (fp8 only)
      packed: kv [B, n_max, d_c + d_R]  (latent in columns [0, d_c), rope after)
      paged : pool [n_pages, page_size, d_c + d_R], block_table int32 [B, n_max/page_size]
    """
    wl: Workload
    lens: np.ndarray
    q_C: np.ndarray
    q_R: np.ndarray
    W_UK: np.ndarray
    W_UV: np.ndarray
    latent: Optional[np.ndarray] = None
    rope: Optional[np.ndarray] = None
    scale: Optional[np.ndarray] = None
    kv: Optional[np.ndarray] = None
    pool: Optional[np.ndarray] = None
    block_table: Optional[np.ndarray] = None
    extra: dict = field(default_factory=dict)

    @property
    def sum_len(self) -> int:
        return int(self.lens.astype(np.int64).sum())

    @property
    def layout(self) -> str:
        return self.wl.layout


def _storage_dtype(kind: str):
    return {"f32": np.float32, "bf16": np.uint16, "fp8": np.uint8}[kind]


def _to_storage(x32: np.ndarray, kind: str) -> np.ndarray:
    if kind == "f32":
        return np.ascontiguousarray(x32, dtype=np.float32)
    return f32_to_bf16_bits(x32)


def _gen_sequence(wl: Workload, child: np.random.SeedSequence, L: int):
    """Latent rows then raw rope rows of one sequence (float32), rope rotated at j."""
    rng = np.random.Generator(np.random.PCG64(child))
    lat = rng.standard_normal((L, wl.d_c), dtype=np.float32)
    raw = rng.standard_normal((L, wl.d_R), dtype=np.float32)
    rope = rope_rotate(raw, np.arange(L), wl.rope_base).astype(np.float32)
    return lat, rope


def make_inputs(wl, seed: Optional[int] = None, poison: bool = True,
                lens: Optional[np.ndarray] = None, threads: Optional[int] = None) -> DecodeInputs:
    """Build the seeded inputs of workload ``wl`` (a Workload, its number or its name).

    ``lens`` overrides the drawn lengths (every other draw is unchanged), which
    tests use for edge cases such as empty or one-token sequences.
    """
    wl = get_workload(wl)
    seed = wl.seed if seed is None else seed
    root = np.random.SeedSequence(seed)
    s_len, s_w, s_q, s_cache, s_page = root.spawn(5)

    B, H, d_h, d_c, d_R, N = wl.B, wl.H, wl.d_h, wl.d_c, wl.d_R, wl.n_max
    r_len = np.random.Generator(np.random.PCG64(s_len))
    drawn = r_len.integers(wl.len_lo, wl.len_hi, size=B, endpoint=True).astype(np.int32)
    if lens is None:
        lens = drawn
    lens = np.asarray(lens, dtype=np.int32).reshape(B)
    if lens.min(initial=0) < 0 or lens.max(initial=0) > N:
        raise ValueError("lengths must lie in [0, n_max]")

    r_w = np.random.Generator(np.random.PCG64(s_w))
    W_UK = (r_w.standard_normal((H, d_h, d_c), dtype=np.float32) * np.float32(wl.w_std))
    W_UV = (r_w.standard_normal((H, d_h, d_c), dtype=np.float32) * np.float32(wl.w_std))

    r_q = np.random.Generator(np.random.PCG64(s_q))
    q_C = r_q.standard_normal((B, H, d_h), dtype=np.float32)
    q_R_raw = r_q.standard_normal((B, H, d_R), dtype=np.float32)
    qpos = np.maximum(lens.astype(np.int64) - 1, 0)[:, None] * np.ones((1, H), dtype=np.int64)
    q_R = rope_rotate(q_R_raw, qpos, wl.rope_base).astype(np.float32)

    qkind = "f32" if wl.dtype == "f32" else "bf16"
    inp = DecodeInputs(wl=wl, lens=lens,
                       q_C=_to_storage(q_C, qkind), q_R=_to_storage(q_R, qkind),
                       W_UK=_to_storage(W_UK, qkind), W_UV=_to_storage(W_UV, qkind))

    children = s_cache.spawn(B)
    lat_kind = wl.dtype
    rope_kind = "f32" if wl.dtype == "f32" else "bf16"
    width = d_c + d_R

    if wl.layout in ("split",):
        lat_store = np.empty((B, N, d_c), dtype=_storage_dtype(lat_kind))
        rope_store = np.empty((B, N, d_R), dtype=_storage_dtype(rope_kind))
        scale_store = np.empty((B, N), dtype=np.float32) if lat_kind == "fp8" else None
    elif wl.layout in ("packed", "paged"):
        if lat_kind != "bf16":
            raise ValueError("packed/paged layouts are bf16")
        kv_store = np.empty((B, N, width), dtype=np.uint16)
    else:
        raise ValueError(wl.layout)

    def fill(b):
        L = int(lens[b])
        lat, rope = _gen_sequence(wl, children[b], L)
        if wl.layout == "split":
            if lat_kind == "fp8":
                codes, sc = quantize_rows_e4m3(lat)
                lat_store[b, :L] = codes
                scale_store[b, :L] = sc
                lat_store[b, L:] = E4M3_NAN if poison else 0
                scale_store[b, L:] = np.nan if poison else 1.0
            else:
                lat_store[b, :L] = _to_storage(lat, lat_kind)
                if lat_kind == "f32":
                    lat_store[b, L:] = np.nan if poison else 0.0
                else:
                    lat_store[b, L:] = BF16_NAN if poison else 0
            rope_store[b, :L] = _to_storage(rope, rope_kind)
            if rope_kind == "f32":
                rope_store[b, L:] = np.nan if poison else 0.0
            else:
                rope_store[b, L:] = BF16_NAN if poison else 0
        else:
            kv_store[b, :L, :d_c] = f32_to_bf16_bits(lat)
            kv_store[b, :L, d_c:] = f32_to_bf16_bits(rope)
            kv_store[b, L:] = BF16_NAN if poison else 0

    nthr = threads if threads is not None else min(8, os.cpu_count() or 1)
    if nthr > 1 and B > 1:
        with _cf.ThreadPoolExecutor(nthr) as ex:
            list(ex.map(fill, range(B)))
    else:
        for b in range(B):
            fill(b)

    if wl.layout == "split":
        inp.latent, inp.rope, inp.scale = lat_store, rope_store, scale_store
    elif wl.layout == "packed":
        inp.kv = kv_store
    else:  # paged
        P = wl.page_size
        if N % P:
            raise ValueError("n_max must be a multiple of the page size")
        pages_per_seq = N // P
        n_pages = B * pages_per_seq
        r_p = np.random.Generator(np.random.PCG64(s_page))
        perm = r_p.permutation(n_pages).astype(np.int32)
        bt = perm.reshape(B, pages_per_seq)
        pool = np.empty((n_pages, P, width), dtype=np.uint16)
        pool[bt.reshape(-1)] = kv_store.reshape(n_pages, P, width)
        inp.pool, inp.block_table = pool, np.ascontiguousarray(bt)
    return inp
