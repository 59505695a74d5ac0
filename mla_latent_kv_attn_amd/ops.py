"""Python binding of the C ABI (include/mla.h) over torch device tensors.

Argument marshalling only: each function passes device pointers, sizes and the current HIP stream
to the function of the same name in libmla_amd.so.  torch provides device memory and streams;
every step of the decode runs in the library's HIP kernels.  There is no fallback: without the
built library every call raises.
"""
from __future__ import annotations

import ctypes
import math
from typing import Optional

import torch

from . import _lib
from ._lib import CacheDesc, MLA_BF16, MLA_F32, MLA_FP8_E4M3, check

_FP8_TYPES = {torch.uint8}
if hasattr(torch, "float8_e4m3fn"):
    _FP8_TYPES.add(torch.float8_e4m3fn)


def dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return MLA_F32
    if t.dtype == torch.bfloat16:
        return MLA_BF16
    if t.dtype in _FP8_TYPES:
        return MLA_FP8_E4M3
    raise TypeError(f"unsupported dtype {t.dtype}")


def _dev(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("tensors must be on a HIP device")


def _scratch(nbytes: int, like: torch.Tensor, stream=None) -> torch.Tensor:
    """A workspace the wrapper allocates itself.  torch frees it when the wrapper returns, while the
    kernels may still be running: on the current stream torch reuses the memory only in stream
    order; on another stream the tensor is recorded on that stream first, so that torch waits for
    its work before reusing the memory."""
    w = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=like.device)
    if stream is not None:
        w.record_stream(stream)
    return w


def _stream(stream, t: torch.Tensor) -> int:
    s = stream if stream is not None else torch.cuda.current_stream(t.device)
    return int(s.cuda_stream)


class Cache:
    """Latent + rope-key cache of one layer, as the mla_cache_desc of include/mla.h.

    Holds references to the tensors so they outlive the descriptor.
    """

    def __init__(self, latent, rope, scale=None, block_table=None, page_size=0):
        _dev(latent, rope, scale, block_table)
        if latent.dim() != 3 or rope.dim() != 3:
            raise ValueError("latent and rope are [B or pages, tokens, width] views")
        if latent.stride(2) != 1 or rope.stride(2) != 1:
            raise ValueError("latent and rope rows must be contiguous")
        self.latent, self.rope, self.scale, self.block_table = latent, rope, scale, block_table
        d = CacheDesc()
        d.latent = latent.data_ptr()
        d.rope = rope.data_ptr()
        d.latent_scale = scale.data_ptr() if scale is not None else None
        d.block_table = block_table.data_ptr() if block_table is not None else None
        d.latent_dtype = dtype_code(latent)
        d.rope_dtype = dtype_code(rope)
        d.latent_stride_b, d.latent_stride_tok = latent.stride(0), latent.stride(1)
        d.rope_stride_b, d.rope_stride_tok = rope.stride(0), rope.stride(1)
        if scale is not None:
            if scale.dtype != torch.float32 or scale.stride(-1) != 1:
                raise ValueError("scale is a float32 [B or pages, tokens] tensor with unit token stride")
            d.scale_stride_b = scale.stride(0)
        if block_table is not None:
            if block_table.dtype != torch.int32 or not block_table.is_contiguous():
                raise ValueError("block_table is a contiguous int32 [B, max_pages] tensor")
            d.page_size = int(page_size)
            d.max_pages = block_table.shape[1]
        self.desc = d

    @classmethod
    def split(cls, latent, rope, scale=None):
        return cls(latent, rope, scale)

    @classmethod
    def packed(cls, kv, d_c: int):
        """kv [B, N, d_c + d_R]: latent in columns [0, d_c), rope key after."""
        return cls(kv[..., :d_c], kv[..., d_c:])

    @classmethod
    def paged(cls, pool, block_table, d_c: int):
        """pool [pages, page_size, d_c + d_R]; block_table [B, max_pages] int32."""
        return cls(pool[..., :d_c], pool[..., d_c:], None, block_table, pool.shape[1])


def mla_absorb_q(q_C: torch.Tensor, W_UK: torch.Tensor, out: Optional[torch.Tensor] = None, stream=None):
    """q'[b,h] = W_UK[h]^T q_C[b,h].  q_C [B,H,d_h], W_UK [H,d_h,d_c]; out [B,H,d_c] (same dtype)."""
    _dev(q_C, W_UK, out)
    B, H, d_h = q_C.shape
    d_c = W_UK.shape[2]
    if out is None:
        out = torch.empty((B, H, d_c), dtype=q_C.dtype, device=q_C.device)
    if not (q_C.is_contiguous() and W_UK.is_contiguous() and out.is_contiguous()):
        raise ValueError("q_C, W_UK and out must be contiguous")
    check("mla_absorb_q", _lib.lib().mla_absorb_q(q_C.data_ptr(), W_UK.data_ptr(), out.data_ptr(), dtype_code(q_C),
                                                  dtype_code(out), B, H, d_h, d_c, _stream(stream, q_C)))
    return out


def mla_decode_workspace_bytes(B: int, H: int, d_c: int, max_len: int, num_splits: int = 0) -> int:
    return int(_lib.lib().mla_decode_workspace_bytes(B, H, d_c, max_len, num_splits))


def mla_decode_auto_splits(B: int, H: int, max_len: int) -> int:
    return int(_lib.lib().mla_decode_auto_splits(B, H, max_len))


def mla_decode_attn(q_abs: torch.Tensor, q_R: torch.Tensor, cache: Cache, seq_lens: torch.Tensor, max_len: int,
                    scale: Optional[float] = None, d_h: Optional[int] = None, num_splits: int = 0,
                    workspace: Optional[torch.Tensor] = None, o_latent: Optional[torch.Tensor] = None,
                    lse: Optional[torch.Tensor] = None, want_lse: bool = True, stream=None):
    """Scores against the cached latents + rope keys, softmax over j < seq_lens[b], latent sum.

    Returns (o_latent [B,H,d_c] float32, lse [B,H] float32 or None).  ``scale`` defaults to
    1/sqrt(d_h + d_R) (``d_h`` then required).
    """
    _dev(q_abs, q_R, seq_lens, workspace, o_latent, lse)
    B, H, d_c = q_abs.shape
    d_R = q_R.shape[2]
    if scale is None:
        if d_h is None:
            raise ValueError("pass scale or d_h")
        scale = 1.0 / math.sqrt(d_h + d_R)
    if seq_lens.dtype != torch.int32 or not seq_lens.is_contiguous():
        raise ValueError("seq_lens is a contiguous int32 [B] tensor")
    if not (q_abs.is_contiguous() and q_R.is_contiguous()):
        raise ValueError("q_abs and q_R must be contiguous")
    need = mla_decode_workspace_bytes(B, H, d_c, max_len, num_splits)
    if workspace is None:
        workspace = _scratch(need, q_abs, stream)
    if o_latent is None:
        o_latent = torch.empty((B, H, d_c), dtype=torch.float32, device=q_abs.device)
    if lse is None and want_lse:
        lse = torch.empty((B, H), dtype=torch.float32, device=q_abs.device)
    st = mla_decode_attn_raw(q_abs, q_R, cache, seq_lens, max_len, scale, num_splits, workspace, o_latent, lse,
                             stream)
    check("mla_decode_attn", st)
    return o_latent, lse


def mla_decode_attn_noalloc(q_abs: torch.Tensor, q_R: torch.Tensor, cache: Cache, seq_lens: torch.Tensor,
                            max_len: int, o_latent: torch.Tensor, lse: Optional[torch.Tensor] = None,
                            scale: Optional[float] = None, d_h: Optional[int] = None, num_splits: int = 0,
                            stream=None):
    """mla_decode_attn with the library's fixed device array as its workspace (include/mla.h):
    writes o_latent [B,H,d_c] (and lse [B,H]); allocates nothing, so o_latent is required."""
    _dev(q_abs, q_R, seq_lens, o_latent, lse)
    B, H, d_c = q_abs.shape
    d_R = q_R.shape[2]
    if scale is None:
        if d_h is None:
            raise ValueError("pass scale or d_h")
        scale = 1.0 / math.sqrt(d_h + d_R)
    check("mla_decode_attn_noalloc", _lib.lib().mla_decode_attn_noalloc(
        q_abs.data_ptr(), q_R.data_ptr(), dtype_code(q_abs), ctypes.byref(cache.desc), seq_lens.data_ptr(),
        int(max_len), B, H, d_c, d_R, float(scale), int(num_splits), o_latent.data_ptr(),
        lse.data_ptr() if lse is not None else None, _stream(stream, q_abs)))
    return o_latent, lse


def mla_decode_attn_raw(q_abs, q_R, cache: Cache, seq_lens, max_len, scale, num_splits, workspace, o_latent, lse,
                        stream=None) -> int:
    """Direct call; returns the status code (used by error-path tests)."""
    B, H, d_c = q_abs.shape
    d_R = q_R.shape[2]
    return _lib.lib().mla_decode_attn(
        q_abs.data_ptr(), q_R.data_ptr(), dtype_code(q_abs), ctypes.byref(cache.desc), seq_lens.data_ptr(),
        int(max_len), B, H, d_c, d_R, float(scale), int(num_splits), workspace.data_ptr(), workspace.numel(),
        o_latent.data_ptr(), lse.data_ptr() if lse is not None else None, _stream(stream, q_abs))


def mla_decode_partial(q_abs, q_R, cache: Cache, seq_lens, max_len: int, scale: float, workspace,
                       num_splits: int = 0, stream=None) -> None:
    """Partial pass of mla_decode_attn into ``workspace`` (see include/mla.h)."""
    _dev(q_abs, q_R, seq_lens, workspace)
    B, H, d_c = q_abs.shape
    d_R = q_R.shape[2]
    check("mla_decode_partial", _lib.lib().mla_decode_partial(
        q_abs.data_ptr(), q_R.data_ptr(), dtype_code(q_abs), ctypes.byref(cache.desc), seq_lens.data_ptr(),
        int(max_len), B, H, d_c, d_R, float(scale), int(num_splits), workspace.data_ptr(), workspace.numel(),
        _stream(stream, q_abs)))


def mla_decode_partial_warm(q_abs, q_R, cache: Cache, seq_lens, max_len: int, scale: float, workspace, warm,
                            num_splits: int = 0, stream=None) -> None:
    """mla_decode_partial that also pulls the device tensor ``warm`` into the last-level cache with
    its spare workgroups (see include/mla.h)."""
    _dev(q_abs, q_R, seq_lens, workspace, warm)
    B, H, d_c = q_abs.shape
    d_R = q_R.shape[2]
    if not warm.is_contiguous():
        raise ValueError("warm must be contiguous")
    check("mla_decode_partial_warm", _lib.lib().mla_decode_partial_warm(
        q_abs.data_ptr(), q_R.data_ptr(), dtype_code(q_abs), ctypes.byref(cache.desc), seq_lens.data_ptr(),
        int(max_len), B, H, d_c, d_R, float(scale), int(num_splits), workspace.data_ptr(), workspace.numel(),
        warm.data_ptr(), warm.numel() * warm.element_size(), _stream(stream, q_abs)))


def mla_decode_combine(seq_lens, max_len: int, B: int, H: int, d_c: int, workspace, o_latent, lse=None,
                       num_splits: int = 0, stream=None) -> None:
    """Combine pass of mla_decode_attn: workspace partials -> o_latent [B,H,d_c], lse [B,H]."""
    _dev(seq_lens, workspace, o_latent, lse)
    check("mla_decode_combine", _lib.lib().mla_decode_combine(
        seq_lens.data_ptr(), int(max_len), B, H, d_c, int(num_splits), workspace.data_ptr(), workspace.numel(),
        o_latent.data_ptr(), lse.data_ptr() if lse is not None else None, _stream(stream, o_latent)))


def mla_decode_combine_uv(seq_lens, max_len: int, workspace, W_UV: torch.Tensor, o_latent: torch.Tensor,
                          out: Optional[torch.Tensor] = None, lse=None, num_splits: int = 0, stream=None):
    """Combine pass + W_UV in one call: workspace partials -> o_latent [B,H,d_c] (and lse [B,H]),
    then out[b,h] = W_UV[h] o_latent[b,h] ([B,H,d_h] float32)."""
    _dev(seq_lens, workspace, W_UV, o_latent, out, lse)
    B, H, d_c = o_latent.shape
    d_h = W_UV.shape[1]
    if out is None:
        out = torch.empty((B, H, d_h), dtype=torch.float32, device=o_latent.device)
    if not (W_UV.is_contiguous() and o_latent.is_contiguous() and out.is_contiguous()):
        raise ValueError("W_UV, o_latent and out must be contiguous")
    check("mla_decode_combine_uv", _lib.lib().mla_decode_combine_uv(
        seq_lens.data_ptr(), int(max_len), B, H, d_c, int(num_splits), workspace.data_ptr(), workspace.numel(),
        W_UV.data_ptr(), dtype_code(W_UV), d_h, out.data_ptr(), o_latent.data_ptr(),
        lse.data_ptr() if lse is not None else None, _stream(stream, o_latent)))
    return out


def mla_uv_out(o_latent: torch.Tensor, W_UV: torch.Tensor, out: Optional[torch.Tensor] = None, stream=None):
    """out[b,h] = W_UV[h] o_latent[b,h].  o_latent [B,H,d_c] float32, W_UV [H,d_h,d_c]; out [B,H,d_h] float32."""
    _dev(o_latent, W_UV, out)
    B, H, d_c = o_latent.shape
    d_h = W_UV.shape[1]
    if out is None:
        out = torch.empty((B, H, d_h), dtype=torch.float32, device=o_latent.device)
    if not (o_latent.is_contiguous() and W_UV.is_contiguous() and out.is_contiguous()):
        raise ValueError("o_latent, W_UV and out must be contiguous")
    check("mla_uv_out", _lib.lib().mla_uv_out(o_latent.data_ptr(), W_UV.data_ptr(), dtype_code(W_UV),
                                              out.data_ptr(), B, H, d_h, d_c, _stream(stream, o_latent)))
    return out


def mla_decode_step_workspace_bytes(B: int, H: int, d_c: int, max_len: int) -> int:
    return int(_lib.lib().mla_decode_step_workspace_bytes(B, H, d_c, max_len))


def mla_decode_step_workspace(B: int, H: int, d_c: int, max_len: int, device) -> torch.Tensor:
    """A zero-filled workspace for mla_decode_step (its flag region must start at zero; every call
    leaves it zero).  The int32 at byte 0 is the sticky error word of the one-launch form."""
    n = mla_decode_step_workspace_bytes(B, H, d_c, max_len)
    return torch.zeros(max(n, 16), dtype=torch.uint8, device=device)


def mla_decode_step_init(workspace: torch.Tensor, stream=None) -> None:
    """Zero the flag region of a step workspace (a fill kernel on the stream)."""
    _dev(workspace)
    check("mla_decode_step_init", _lib.lib().mla_decode_step_init(workspace.data_ptr(), workspace.numel(),
                                                                  _stream(stream, workspace)))


def mla_decode_step(q_C, q_R, W_UK, W_UV, cache: Cache, seq_lens, max_len: int, workspace: torch.Tensor,
                    out: Optional[torch.Tensor] = None, q_abs: Optional[torch.Tensor] = None,
                    o_latent: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                    scale: Optional[float] = None, stream=None) -> torch.Tensor:
    """The whole absorbed decode step (include/mla.h, mla_decode_step): out [B,H,d_h] fp32 from
    q_C [B,H,d_h], q_R [B,H,d_R], W_UK / W_UV [H,d_h,d_c] and the cache.  q_abs, o_latent and lse
    are written when given.  ``workspace`` comes from mla_decode_step_workspace (zero-filled)."""
    _dev(q_C, q_R, W_UK, W_UV, seq_lens, workspace, out, q_abs, o_latent, lse)
    B, H, d_h = q_C.shape
    d_R = q_R.shape[2]
    d_c = W_UK.shape[2]
    if scale is None:
        scale = 1.0 / math.sqrt(d_h + d_R)
    if out is None:
        out = torch.empty((B, H, d_h), dtype=torch.float32, device=q_C.device)
    for t in (q_C, q_R, W_UK, W_UV, out, q_abs, o_latent, lse):
        if t is not None and not t.is_contiguous():
            raise ValueError("mla_decode_step takes contiguous tensors")
    if q_abs is not None and q_abs.dtype != q_C.dtype:
        raise ValueError("q_abs has the dtype of q_C")

    def ptr(t):
        return t.data_ptr() if t is not None else None

    check("mla_decode_step", _lib.lib().mla_decode_step(
        q_C.data_ptr(), q_R.data_ptr(), W_UK.data_ptr(), W_UV.data_ptr(), dtype_code(q_C), ctypes.byref(cache.desc),
        seq_lens.data_ptr(), int(max_len), B, H, d_h, d_c, d_R, float(scale), workspace.data_ptr(),
        workspace.numel(), ptr(q_abs), ptr(o_latent), ptr(lse), out.data_ptr(), _stream(stream, q_C)))
    return out


def mla_cache_append_workspace_bytes(B: int, D: int) -> int:
    return int(_lib.lib().mla_cache_append_workspace_bytes(B, D))


def mla_cache_append(h: torch.Tensor, W_DKV: torch.Tensor, W_KR: torch.Tensor, pos: torch.Tensor, cache: Cache,
                     rope_base: float = 10000.0, workspace: Optional[torch.Tensor] = None, stream=None) -> None:
    """Write each sequence's new token into cache row pos[b]: latent W_DKV h[b], rope key
    RoPE_pos[b](W_KR h[b]).  h [B, D] bf16, W_DKV [d_c, D], W_KR [d_R, D] bf16, pos [B] int32."""
    _dev(h, W_DKV, W_KR, pos, workspace)
    B, D = h.shape
    d_c, d_R = W_DKV.shape[0], W_KR.shape[0]
    if not (h.is_contiguous() and W_DKV.is_contiguous() and W_KR.is_contiguous() and pos.is_contiguous()):
        raise ValueError("h, W_DKV, W_KR and pos must be contiguous")
    if pos.dtype != torch.int32:
        raise TypeError("pos is int32")
    if workspace is None:
        workspace = _scratch(mla_cache_append_workspace_bytes(B, D), h, stream)
    check("mla_cache_append", _lib.lib().mla_cache_append(
        h.data_ptr(), W_DKV.data_ptr(), W_KR.data_ptr(), dtype_code(h), pos.data_ptr(), ctypes.byref(cache.desc), B,
        D, d_c, d_R, float(rope_base), workspace.data_ptr(), workspace.numel(), _stream(stream, h)))


def mla_proj_workspace_bytes(B: int, N: int, K: int) -> int:
    return int(_lib.lib().mla_proj_workspace_bytes(B, N, K))


def mla_query_workspace_bytes(B: int, D: int, d_q: int, H: int, d_h: int, d_R: int) -> int:
    return int(_lib.lib().mla_query_workspace_bytes(B, D, d_q, H, d_h, d_R))


def _contig(**ts):
    for name, t in ts.items():
        if t is not None and not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")


def _ws(nbytes: int, like: torch.Tensor, workspace: Optional[torch.Tensor], stream=None):
    """(address, size) of the workspace: the caller's, else a fresh one of nbytes (none when 0)."""
    if workspace is not None:
        return workspace.data_ptr(), workspace.numel() * workspace.element_size()
    if nbytes == 0:
        return 0, 0
    w = _scratch(nbytes, like, stream)
    return w.data_ptr(), nbytes


def mla_query_proj(h: torch.Tensor, W_DQ: torch.Tensor, W_UQ: torch.Tensor, W_QR: torch.Tensor, pos: torch.Tensor,
                   H: int, rope_base: float = 10000.0, c_q: Optional[torch.Tensor] = None,
                   q_C: Optional[torch.Tensor] = None, q_R: Optional[torch.Tensor] = None,
                   workspace: Optional[torch.Tensor] = None, stream=None):
    """c_q = W_DQ h, q_C = W_UQ c_q, q_R = RoPE_pos(W_QR c_q) per head.  h [B, D] bf16,
    W_DQ [d_q, D], W_UQ [H d_h, d_q], W_QR [H d_R, d_q] bf16, pos [B] int32.
    Returns (c_q [B, d_q], q_C [B, H, d_h], q_R [B, H, d_R]), all bf16."""
    _dev(h, W_DQ, W_UQ, W_QR, pos, c_q, q_C, q_R, workspace)
    _contig(h=h, W_DQ=W_DQ, W_UQ=W_UQ, W_QR=W_QR, pos=pos, c_q=c_q, q_C=q_C, q_R=q_R)
    if pos.dtype != torch.int32:
        raise TypeError("pos is int32")
    B, D = h.shape
    d_q = W_DQ.shape[0]
    d_h, d_R = W_UQ.shape[0] // H, W_QR.shape[0] // H
    if c_q is None:
        c_q = torch.empty(B, d_q, dtype=torch.bfloat16, device=h.device)
    if q_C is None:
        q_C = torch.empty(B, H, d_h, dtype=torch.bfloat16, device=h.device)
    if q_R is None:
        q_R = torch.empty(B, H, d_R, dtype=torch.bfloat16, device=h.device)
    wp, wn = _ws(mla_query_workspace_bytes(B, D, d_q, H, d_h, d_R), h, workspace, stream)
    check("mla_query_proj", _lib.lib().mla_query_proj(
        h.data_ptr(), W_DQ.data_ptr(), W_UQ.data_ptr(), W_QR.data_ptr(), dtype_code(h), pos.data_ptr(), B, D, d_q,
        H, d_h, d_R, float(rope_base), c_q.data_ptr(), q_C.data_ptr(), q_R.data_ptr(), wp, wn, _stream(stream, h)))
    return c_q, q_C, q_R


def mla_query_append_workspace_bytes(B: int, D: int, d_q: int, H: int, d_h: int, d_R: int, d_c: int) -> int:
    return int(_lib.lib().mla_query_append_workspace_bytes(B, D, d_q, H, d_h, d_R, d_c))


def mla_query_proj_append(h: torch.Tensor, W_DQ: torch.Tensor, W_UQ: torch.Tensor, W_QR: torch.Tensor,
                          W_DKV: torch.Tensor, W_KR: torch.Tensor, pos: torch.Tensor, cache: Cache, H: int,
                          rope_base: float = 10000.0, c_q: Optional[torch.Tensor] = None,
                          q_C: Optional[torch.Tensor] = None, q_R: Optional[torch.Tensor] = None,
                          workspace: Optional[torch.Tensor] = None, stream=None):
    """mla_query_proj and mla_cache_append of the same tokens in two projections (bf16 caches).
    Returns (c_q, q_C, q_R) as mla_query_proj; the cache row pos[b] is written as mla_cache_append."""
    _dev(h, W_DQ, W_UQ, W_QR, W_DKV, W_KR, pos, c_q, q_C, q_R, workspace)
    _contig(h=h, W_DQ=W_DQ, W_UQ=W_UQ, W_QR=W_QR, W_DKV=W_DKV, W_KR=W_KR, pos=pos, c_q=c_q, q_C=q_C, q_R=q_R)
    if pos.dtype != torch.int32:
        raise TypeError("pos is int32")
    B, D = h.shape
    d_q, d_c, d_R = W_DQ.shape[0], W_DKV.shape[0], W_KR.shape[0]
    d_h = W_UQ.shape[0] // H
    if W_QR.shape[0] != H * d_R:
        raise ValueError("W_QR rows must be H * d_R (the rope width of W_KR)")
    if c_q is None:
        c_q = torch.empty(B, d_q, dtype=torch.bfloat16, device=h.device)
    if q_C is None:
        q_C = torch.empty(B, H, d_h, dtype=torch.bfloat16, device=h.device)
    if q_R is None:
        q_R = torch.empty(B, H, d_R, dtype=torch.bfloat16, device=h.device)
    wp, wn = _ws(mla_query_append_workspace_bytes(B, D, d_q, H, d_h, d_R, d_c), h, workspace, stream)
    check("mla_query_proj_append", _lib.lib().mla_query_proj_append(
        h.data_ptr(), W_DQ.data_ptr(), W_UQ.data_ptr(), W_QR.data_ptr(), W_DKV.data_ptr(), W_KR.data_ptr(),
        dtype_code(h), pos.data_ptr(), ctypes.byref(cache.desc), B, D, d_q, H, d_h, d_R, d_c, float(rope_base),
        c_q.data_ptr(), q_C.data_ptr(), q_R.data_ptr(), wp, wn, _stream(stream, h)))
    return c_q, q_C, q_R


def mla_fold_q(W_UQ: torch.Tensor, W_UK: torch.Tensor, out: Optional[torch.Tensor] = None, stream=None):
    """W_QK[h] = W_UK[h]^T W_UQ[h d_h:(h+1) d_h]: W_UQ [H d_h, d_q], W_UK [H, d_h, d_c] -> [H, d_c, d_q] bf16."""
    _dev(W_UQ, W_UK, out)
    _contig(W_UQ=W_UQ, W_UK=W_UK, out=out)
    H, d_h, d_c = W_UK.shape
    d_q = W_UQ.shape[1]
    if out is None:
        out = torch.empty(H, d_c, d_q, dtype=torch.bfloat16, device=W_UK.device)
    check("mla_fold_q", _lib.lib().mla_fold_q(W_UQ.data_ptr(), W_UK.data_ptr(), dtype_code(W_UK), out.data_ptr(),
                                              H, d_h, d_c, d_q, _stream(stream, W_UK)))
    return out


def mla_absorb_q_folded(c_q: torch.Tensor, W_QK: torch.Tensor, out: Optional[torch.Tensor] = None,
                        out_dtype=torch.bfloat16, workspace: Optional[torch.Tensor] = None, stream=None):
    """q'[b, h] = W_QK[h] c_q[b]: c_q [B, d_q] bf16, W_QK [H, d_c, d_q] bf16 -> [B, H, d_c]."""
    _dev(c_q, W_QK, out, workspace)
    _contig(c_q=c_q, W_QK=W_QK, out=out)
    B, d_q = c_q.shape
    H, d_c = W_QK.shape[0], W_QK.shape[1]
    if out is None:
        out = torch.empty(B, H, d_c, dtype=out_dtype, device=c_q.device)
    wp, wn = _ws(mla_proj_workspace_bytes(B, H * d_c, d_q), c_q, workspace, stream)
    check("mla_absorb_q_folded", _lib.lib().mla_absorb_q_folded(
        c_q.data_ptr(), W_QK.data_ptr(), dtype_code(c_q), out.data_ptr(), dtype_code(out), B, H, d_c, d_q, wp, wn,
        _stream(stream, c_q)))
    return out


def mla_out_proj(x: torch.Tensor, W: torch.Tensor, out: Optional[torch.Tensor] = None,
                 workspace: Optional[torch.Tensor] = None, stream=None):
    """out[b] = W x[b]: x [B, ...] float32 (flattened to [B, K]), W [D, K] bf16 -> [B, D] float32."""
    _dev(x, W, out, workspace)
    _contig(x=x, W=W, out=out)
    if x.dtype != torch.float32:
        raise TypeError("x is float32")
    B = x.shape[0]
    K = x.numel() // max(B, 1)
    D = W.shape[0]
    if W.shape[1] != K:
        raise ValueError(f"W has {W.shape[1]} columns, x has {K} values per token")
    if out is None:
        out = torch.empty(B, D, dtype=torch.float32, device=x.device)
    wp, wn = _ws(mla_proj_workspace_bytes(B, D, K), x, workspace, stream)
    check("mla_out_proj", _lib.lib().mla_out_proj(x.data_ptr(), W.data_ptr(), dtype_code(W), out.data_ptr(), B, D,
                                                  K, wp, wn, _stream(stream, x)))
    return out


def mla_fold_o(W_O: torch.Tensor, W_UV: torch.Tensor, out: Optional[torch.Tensor] = None, stream=None):
    """W_OV[:, h d_c:(h+1) d_c] = W_O[:, h d_h:(h+1) d_h] W_UV[h]: W_O [D, H d_h], W_UV [H, d_h, d_c]
    -> [D, H d_c] bf16."""
    _dev(W_O, W_UV, out)
    _contig(W_O=W_O, W_UV=W_UV, out=out)
    H, d_h, d_c = W_UV.shape
    D = W_O.shape[0]
    if out is None:
        out = torch.empty(D, H * d_c, dtype=torch.bfloat16, device=W_O.device)
    check("mla_fold_o", _lib.lib().mla_fold_o(W_O.data_ptr(), W_UV.data_ptr(), dtype_code(W_O), out.data_ptr(), D,
                                              H, d_h, d_c, _stream(stream, W_O)))
    return out


def mla_mha_decode_workspace_bytes(B: int, H: int, max_len: int, num_splits: int = 0) -> int:
    return int(_lib.lib().mla_mha_decode_workspace_bytes(B, H, max_len, num_splits))


def mla_mha_decode(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, seq_lens: torch.Tensor,
                   max_len: int, scale: Optional[float] = None, num_splits: int = 0, workspace=None, out=None,
                   lse=None, stream=None) -> torch.Tensor:
    """Same-dimension MHA decode (comparison path): q [B,H,192], k_cache [B,H,cap,192],
    v_cache [B,H,cap,128] bf16 -> out [B,H,128] float32."""
    _dev(q, k_cache, v_cache, seq_lens, workspace, out, lse)
    B, H, d_k = q.shape
    cap, d_v = k_cache.shape[2], v_cache.shape[3]
    if not (q.is_contiguous() and k_cache.is_contiguous() and v_cache.is_contiguous()):
        raise ValueError("q, k_cache and v_cache must be contiguous")
    if scale is None:
        scale = 1.0 / math.sqrt(d_k)
    if out is None:
        out = torch.empty((B, H, d_v), dtype=torch.float32, device=q.device)
    if workspace is None:
        workspace = _scratch(mla_mha_decode_workspace_bytes(B, H, max_len, num_splits), q, stream)
    check("mla_mha_decode", _lib.lib().mla_mha_decode(
        q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), dtype_code(q), seq_lens.data_ptr(), int(max_len), cap,
        B, H, d_k, d_v, float(scale), int(num_splits), workspace.data_ptr(), workspace.numel(), out.data_ptr(),
        lse.data_ptr() if lse is not None else None, _stream(stream, q)))
    return out
