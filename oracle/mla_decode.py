"""Plain CPU reference of one MLA decode step (test infrastructure only).

Definitions followed (cited by page title and section):

* Keys and values are rebuilt from the cached latent by per-head
  up-projections, k_C = W_UK c and v_C = W_UV c (column-vector form), as in
  "Grouped-query and latent attention", section "Multi-head latent attention
  (MLA)"; the row-vector form of "MLA storage: Representing KV with a small
  latent vector", section "Forming head-specific K and V from a small vector",
  is its transpose.
* The full key of a head is the concatenation [k_C ; k_R] with the shared,
  already rotated rope key k_R, and the query is [q_C ; q_R]
  ("Grouped-query and latent attention", section "Why a separate rotary key";
  "MLA storage ...", section "Two paths for forming keys and values", which
  also states the rope key is not appended to the value).
* Scores are scaled by 1/sqrt(d_h + d_R) (same section: 1/sqrt(128 + 64)).
* The attention row of the newest token is Softmax(q K^T) and the context
  vector is that row times V ("The Journey to Multi-Head Latent Attention",
  section "The KV cache -- and why it exists at all", step 2).
* A decode query sees every cached row j < len_b; padding rows are never read.

Storage decoding (bf16 bit patterns, OCP E4M3 codes with a per-token float32
scale) is written here from the formats' definitions and shares nothing with
the input generator's encoders or with the GPU kernels.
"""
from __future__ import annotations

import math
from typing import Iterable, Optional, Sequence, Tuple

import numpy as np


# --------------------------------------------------------------------------
# storage decoding
# --------------------------------------------------------------------------
def decode_bf16(bits) -> np.ndarray:
    """bfloat16 bit patterns -> float64 (exact): the 16 bits are the top half of a float32."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def _e4m3_value(code: int) -> float:
    """Value of one OCP FP8 E4M3 code: sign, 4 exponent bits (bias 7), 3 mantissa bits.

    Exponent field 0 is subnormal (m/8 * 2**-6); S.1111.111 is NaN; there is no infinity.
    """
    s = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return math.nan
    if e == 0:
        return s * (m / 8.0) * 2.0 ** -6
    return s * (1.0 + m / 8.0) * 2.0 ** (e - 7)


_E4M3_TABLE = np.array([_e4m3_value(c) for c in range(256)], dtype=np.float64)


def decode_e4m3(codes, scale=None) -> np.ndarray:
    """E4M3 codes (uint8) -> float64; multiplied by a per-row scale when given."""
    v = _E4M3_TABLE[np.asarray(codes, dtype=np.uint8)]
    if scale is not None:
        v = v * np.asarray(scale, dtype=np.float64)[..., None]
    return v


def _as_real(a, kind: str) -> np.ndarray:
    if kind == "f32":
        return np.asarray(a, dtype=np.float64)
    if kind == "bf16":
        return decode_bf16(a)
    raise ValueError(kind)


def _kind(inp) -> Tuple[str, str]:
    """(storage kind of queries/weights/rope, storage kind of latents)."""
    lat = inp.wl.dtype
    other = "f32" if lat == "f32" else "bf16"
    return other, lat


# --------------------------------------------------------------------------
# cache read: the rows a decode query attends to
# --------------------------------------------------------------------------
def gather_rows(inp, b: int) -> Tuple[np.ndarray, np.ndarray]:
    """Latent rows C_b [len_b, d_c] and rope rows R_b [len_b, d_R] of sequence b, float64.

    split : C = latent[b, :L], R = rope[b, :L]   (fp8: C = scale_j * e4m3(latent[b, j]))
    packed: C = kv[b, :L, :d_c], R = kv[b, :L, d_c:]
    paged : row j lives in page block_table[b, j // P] at slot j % P of the pool
    """
    wl = inp.wl
    L = int(inp.lens[b])
    d_c = wl.d_c
    other, lat = _kind(inp)
    if wl.layout == "split":
        if lat == "fp8":
            C = decode_e4m3(inp.latent[b, :L], inp.scale[b, :L])
        else:
            C = _as_real(inp.latent[b, :L], lat)
        R = _as_real(inp.rope[b, :L], other)
    elif wl.layout == "packed":
        rows = decode_bf16(inp.kv[b, :L])
        C, R = rows[:, :d_c], rows[:, d_c:]
    elif wl.layout == "paged":
        P = wl.page_size
        j = np.arange(L)
        pages = inp.block_table[b, j // P]
        rows = decode_bf16(inp.pool[pages, j % P])
        C, R = rows[:, :d_c], rows[:, d_c:]
    else:
        raise ValueError(wl.layout)
    return C, R


# --------------------------------------------------------------------------
# the definition
# --------------------------------------------------------------------------
def expand_kv(C_b: np.ndarray, R_b: np.ndarray, W_UK_h: np.ndarray, W_UV_h: np.ndarray):
    """Explicit per-head keys and values of every cached token.

    K[j] = [W_UK_h c_j ; k_R,j]  (length d_h + d_R),   V[j] = W_UV_h c_j  (length d_h).
    W_UK_h and W_UV_h are [d_h, d_c] (column-vector form: k_C = W_UK_h c).
    """
    K_C = C_b @ W_UK_h.T
    K = np.concatenate([K_C, R_b], axis=1)
    V = C_b @ W_UV_h.T
    return K, V


def attend(K: np.ndarray, V: np.ndarray, q: np.ndarray, scale: float):
    """Softmax attention of one query over rows of K/V (two-pass, max-subtracted).

    Returns (o, lse, a): output, log-sum-exp of the scaled scores, and the weights.
    An empty K gives o = 0, lse = -inf.
    """
    L = K.shape[0]
    if L == 0:
        return np.zeros(V.shape[1], dtype=K.dtype), -math.inf, np.zeros(0, dtype=K.dtype)
    s = (K @ q) * scale
    mx = np.max(s)
    e = np.exp(s - mx)
    tot = np.sum(e)
    a = e / tot
    o = a @ V
    lse = float(mx + np.log(tot))
    return o, lse, a


def decode(inp, pairs: Optional[Iterable[Tuple[int, int]]] = None, dtype=np.float64,
           want_diag: bool = True) -> dict:
    """Reference decode step.

    Returns a dict of arrays (NaN where a (b, h) pair was not requested):
      o      [B, H, d_h]  attention output per head (after W_UV)
      lse    [B, H]       natural-log log-sum-exp of the scaled scores
      q_abs  [B, H, d_c]  W_UK[h]^T q_C[b, h]          (diagnostic for mla_absorb_q)
      o_lat  [B, H, d_c]  sum_j a_j c_j                 (diagnostic for mla_decode_attn)
    """
    wl = inp.wl
    B, H, d_h, d_c, d_R = wl.B, wl.H, wl.d_h, wl.d_c, wl.d_R
    other, _ = _kind(inp)
    scale = 1.0 / math.sqrt(d_h + d_R)
    q_C = _as_real(inp.q_C, other).astype(dtype)
    q_R = _as_real(inp.q_R, other).astype(dtype)
    W_UK = _as_real(inp.W_UK, other).astype(dtype)
    W_UV = _as_real(inp.W_UV, other).astype(dtype)

    if pairs is None:
        pairs = [(b, h) for b in range(B) for h in range(H)]
    by_b = {}
    for b, h in pairs:
        by_b.setdefault(int(b), []).append(int(h))

    o = np.full((B, H, d_h), np.nan)
    lse = np.full((B, H), np.nan)
    q_abs = np.full((B, H, d_c), np.nan) if want_diag else None
    o_lat = np.full((B, H, d_c), np.nan) if want_diag else None

    for b, heads in by_b.items():
        C_b, R_b = gather_rows(inp, b)
        C_b = C_b.astype(dtype)
        R_b = R_b.astype(dtype)
        for h in heads:
            K, V = expand_kv(C_b, R_b, W_UK[h], W_UV[h])
            q = np.concatenate([q_C[b, h], q_R[b, h]])
            o_bh, lse_bh, a = attend(K, V, q, scale)
            o[b, h] = o_bh
            lse[b, h] = lse_bh
            if want_diag:
                q_abs[b, h] = W_UK[h].T @ q_C[b, h]
                o_lat[b, h] = a @ C_b if C_b.shape[0] else 0.0
    return {"o": o, "lse": lse, "q_abs": q_abs, "o_lat": o_lat}


# --------------------------------------------------------------------------
# split-N merge (the combine pass, as a definition)
# --------------------------------------------------------------------------
def merge_partials(ms: Sequence[float], ls: Sequence[float], accs: Sequence[np.ndarray]):
    """Merge per-split softmax partials of one (sequence, head).

    Split s holds m_s = max of its scaled scores, l_s = sum exp(s_j - m_s) and
    acc_s = sum exp(s_j - m_s) x_j (empty split: m_s = -inf, l_s = 0, acc_s = 0).
    Result: M = max m_s, L = sum exp(m_s - M) l_s, out = sum exp(m_s - M) acc_s / L,
    lse = M + log L.  All splits empty gives out = 0, lse = -inf.
    """
    ms = np.asarray(ms, dtype=np.float64)
    ls = np.asarray(ls, dtype=np.float64)
    accs = np.asarray(accs, dtype=np.float64)
    if ms.size == 0 or not np.isfinite(ms).any():
        return np.zeros(accs.shape[-1]), -math.inf
    M = np.max(ms[np.isfinite(ms)])
    w = np.where(np.isfinite(ms), np.exp(np.where(np.isfinite(ms), ms, M) - M), 0.0)
    Ltot = float(np.sum(w * ls))
    out = (w[:, None] * accs).sum(axis=0) / Ltot
    return out, float(M + math.log(Ltot))


def relative_l2(x, ref) -> float:
    """||x - ref||_2 / ||ref||_2 over all finite-reference entries (NaN entries of ref skipped)."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    m = ~np.isnan(ref)
    num = np.linalg.norm((x - ref)[m])
    den = np.linalg.norm(ref[m])
    if den == 0.0:
        return float(num)
    return float(num / den)
