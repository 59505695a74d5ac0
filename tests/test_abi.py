"""C-ABI checks that need no GPU: the library loads, exports every declared function, and rejects
invalid arguments with the documented status before launching anything.

Pointers passed here are never dereferenced: each call fails host-side validation first (or is a
documented no-op such as B == 0).
"""
from __future__ import annotations

import ctypes
import math

import pytest

from mla_latent_kv_attn_amd import _lib as L

FAKE = 0x10000  # 16-byte aligned, never dereferenced


@pytest.fixture(scope="module")
def lib():
    return L.lib()


def test_library_exports_every_declared_function(lib):
    names = L.header_functions()
    assert {"mla_absorb_q", "mla_decode_attn", "mla_uv_out", "mla_decode_workspace_bytes"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n
    assert lib.mla_version() == 10000
    assert lib.mla_last_hip_error() == 0


def test_status_strings(lib):
    for code in range(7):
        s = lib.mla_status_string(code).decode()
        assert s.startswith("MLA_")
    assert "unknown" in lib.mla_status_string(99).decode()


def test_absorb_validation(lib):
    f = lib.mla_absorb_q
    assert f(FAKE, FAKE, FAKE, L.MLA_BF16, L.MLA_BF16, -1, 128, 128, 512, None) == L.MLA_ERR_SHAPE
    assert f(FAKE, FAKE, FAKE, L.MLA_BF16, L.MLA_BF16, 1, 0, 128, 512, None) == L.MLA_ERR_SHAPE
    assert f(FAKE, FAKE, FAKE, 9, L.MLA_BF16, 1, 128, 128, 512, None) == L.MLA_ERR_DTYPE
    assert f(None, None, None, L.MLA_BF16, L.MLA_BF16, 0, 128, 128, 512, None) == L.MLA_OK   # no-op
    assert f(None, FAKE, FAKE, L.MLA_BF16, L.MLA_BF16, 1, 128, 128, 512, None) == L.MLA_ERR_NULL
    assert f(FAKE, FAKE, FAKE, L.MLA_BF16, L.MLA_BF16, 1, 128, 64, 512, None) == L.MLA_ERR_UNSUPPORTED
    assert f(FAKE, FAKE, FAKE, L.MLA_F32, L.MLA_BF16, 1, 128, 128, 512, None) == L.MLA_ERR_UNSUPPORTED
    assert f(FAKE, FAKE, FAKE, L.MLA_F32, L.MLA_F32, 1, 4, 16, 8192, None) == L.MLA_ERR_UNSUPPORTED
    assert f(FAKE + 2, FAKE, FAKE, L.MLA_BF16, L.MLA_BF16, 1, 128, 128, 512, None) == L.MLA_ERR_UNSUPPORTED


def test_workspace_size_formula(lib):
    ws = lib.mla_decode_workspace_bytes
    assert ws(0, 128, 512, 4096, 0) == 0 and ws(1, 128, 512, -1, 0) == 0 and ws(1, 128, 512, 64, -2) == 0
    for B, H, d_c, N, S in [(1, 128, 512, 4096, 0), (64, 128, 512, 8192, 0), (3, 4, 32, 64, 7), (16, 64, 512, 100, 1)]:
        W = S if S else lib.mla_decode_auto_splits(B, H, N)
        slots = W + B - 1
        acc = (slots * H * d_c * 4 + 255) // 256 * 256
        ml = (slots * H * 2 * 4 + 255) // 256 * 256
        prefix = ((B + 2) * 4 + 255) // 256 * 256   # tile prefix sums and the partial sums' format
        cnt = (H * 4 + 255) // 256 * 256
        uv = (min(B, 4) * H * 4 * 128 * 4 + 255) // 256 * 256
        assert ws(B, H, d_c, N, S) == acc + ml + prefix + cnt + uv
    # the auto choice: up to 1024 tiles of 32 tokens in total, ceil(3 T / 8) splits, at most 64;
    # beyond that about two tiles per split, at most 256
    assert lib.mla_decode_auto_splits(1, 128, 4096) == 48
    assert lib.mla_decode_auto_splits(1, 128, 4095) == 48
    assert lib.mla_decode_auto_splits(1, 128, 64) == 1
    assert lib.mla_decode_auto_splits(1, 128, 96) == 2
    assert lib.mla_decode_auto_splits(32, 128, 1024) == 64
    assert lib.mla_decode_auto_splits(33, 128, 1024) == 256
    assert lib.mla_decode_auto_splits(8, 128, 1024) == 64
    assert lib.mla_decode_auto_splits(64, 128, 8192) == 256
    assert lib.mla_decode_auto_splits(1, 128, 1) == 1


def _desc(latent_dtype=L.MLA_BF16, rope_dtype=L.MLA_BF16, scale=None, bt=None, page=0, max_pages=0,
          latent=FAKE, st_tok=576, st_b=576 * 4096, rope_st=576):
    d = L.CacheDesc()
    d.latent, d.rope = latent, FAKE + 1024
    d.latent_scale, d.block_table = scale, bt
    d.latent_dtype, d.rope_dtype = latent_dtype, rope_dtype
    d.latent_stride_b, d.latent_stride_tok = st_b, st_tok
    d.rope_stride_b, d.rope_stride_tok = st_b, rope_st
    d.scale_stride_b = 4096
    d.page_size, d.max_pages = page, max_pages
    return d


def _attn(lib, desc, B=1, H=128, d_c=512, d_R=64, q_dtype=L.MLA_BF16, max_len=4096, scale=1 / math.sqrt(192),
          splits=0, ws=FAKE, ws_bytes=1 << 40, q=FAKE, lens=FAKE, out=FAKE):
    return lib.mla_decode_attn(q, FAKE, q_dtype, ctypes.byref(desc) if desc is not None else None, lens, max_len, B,
                               H, d_c, d_R, scale, splits, ws, ws_bytes, out, None, None)


def test_decode_attn_validation(lib):
    d = _desc()
    assert _attn(lib, d, B=-1) == L.MLA_ERR_SHAPE
    assert _attn(lib, d, d_c=6) == L.MLA_ERR_SHAPE
    assert _attn(lib, d, max_len=-5) == L.MLA_ERR_SHAPE
    assert _attn(lib, d, scale=float("nan")) == L.MLA_ERR_SHAPE
    assert _attn(lib, d, B=3000) == L.MLA_ERR_UNSUPPORTED
    assert _attn(lib, d, B=2049) == L.MLA_ERR_UNSUPPORTED                # the batch limit is 2048
    assert _attn(lib, None) == L.MLA_ERR_NULL
    assert _attn(lib, d, q_dtype=7) == L.MLA_ERR_DTYPE
    assert _attn(lib, _desc(latent_dtype=5)) == L.MLA_ERR_DTYPE
    assert _attn(lib, d, B=0) == L.MLA_OK                                # no-op
    assert _attn(lib, d, q=None) == L.MLA_ERR_NULL
    assert _attn(lib, d, lens=None) == L.MLA_ERR_NULL
    assert _attn(lib, d, ws=None) == L.MLA_ERR_WORKSPACE
    need = lib.mla_decode_workspace_bytes(1, 128, 512, 4096, 0)
    assert _attn(lib, d, ws_bytes=need - 1) == L.MLA_ERR_WORKSPACE
    assert _attn(lib, d, ws=FAKE + 8) == L.MLA_ERR_UNSUPPORTED           # workspace not 16-byte aligned
    assert _attn(lib, d, out=FAKE + 4) == L.MLA_ERR_UNSUPPORTED          # o_latent not 16-byte aligned
    assert _attn(lib, d, d_c=256) == L.MLA_ERR_UNSUPPORTED               # bf16 path is d_c = 512 only
    assert _attn(lib, d, H=96) == L.MLA_ERR_UNSUPPORTED
    assert _attn(lib, _desc(latent=FAKE + 2)) == L.MLA_ERR_UNSUPPORTED   # misaligned rows
    assert _attn(lib, _desc(st_tok=577)) == L.MLA_ERR_UNSUPPORTED
    assert _attn(lib, _desc(latent_dtype=L.MLA_FP8_E4M3)) == L.MLA_ERR_NULL   # fp8 needs scales
    assert _attn(lib, _desc(latent_dtype=L.MLA_F32, rope_dtype=L.MLA_F32)) == L.MLA_ERR_UNSUPPORTED
    assert _attn(lib, _desc(bt=FAKE, page=48, max_pages=100)) == L.MLA_ERR_UNSUPPORTED
    assert _attn(lib, _desc(bt=FAKE, page=64, max_pages=10)) == L.MLA_ERR_SHAPE   # 640 < max_len
    assert _attn(lib, _desc(bt=FAKE, page=0, max_pages=10)) == L.MLA_ERR_SHAPE
    assert _attn(lib, _desc(latent_dtype=L.MLA_F32, rope_dtype=L.MLA_F32), q_dtype=L.MLA_F32, d_c=2048) == \
        L.MLA_ERR_UNSUPPORTED


def test_uv_out_validation(lib):
    f = lib.mla_uv_out
    assert f(FAKE, FAKE, L.MLA_BF16, FAKE, -1, 128, 128, 512, None) == L.MLA_ERR_SHAPE
    assert f(FAKE, FAKE, 5, FAKE, 1, 128, 128, 512, None) == L.MLA_ERR_DTYPE
    assert f(None, FAKE, L.MLA_BF16, FAKE, 1, 128, 128, 512, None) == L.MLA_ERR_NULL
    assert f(None, None, L.MLA_BF16, None, 0, 128, 128, 512, None) == L.MLA_OK
    assert f(FAKE, FAKE, L.MLA_FP8_E4M3, FAKE, 1, 128, 128, 512, None) == L.MLA_ERR_UNSUPPORTED


def test_binding_raises_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(L, "_lib", None)
    monkeypatch.setattr(L, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(L.MlaLibraryError):
        L.lib()


def test_combine_uv_validation(lib):
    f = lib.mla_decode_combine_uv
    need = lib.mla_decode_workspace_bytes(1, 128, 512, 4096, 0)
    args = dict(lens=FAKE, max_len=4096, B=1, H=128, d_c=512, splits=0, ws=FAKE, ws_bytes=need, w=FAKE,
                w_dtype=L.MLA_BF16, d_h=128, out=FAKE, o_lat=FAKE, lse=None)

    def call(**kw):
        a = dict(args, **kw)
        return f(a["lens"], a["max_len"], a["B"], a["H"], a["d_c"], a["splits"], a["ws"], a["ws_bytes"], a["w"],
                 a["w_dtype"], a["d_h"], a["out"], a["o_lat"], a["lse"], None)
    assert call(B=-1) == L.MLA_ERR_SHAPE
    assert call(d_h=0) == L.MLA_ERR_SHAPE
    assert call(w_dtype=9) == L.MLA_ERR_DTYPE
    assert call(ws=None) == L.MLA_ERR_WORKSPACE
    assert call(ws_bytes=need - 1) == L.MLA_ERR_WORKSPACE
    assert call(o_lat=None) == L.MLA_ERR_NULL
    assert call(w=None) == L.MLA_ERR_NULL
    assert call(out=None) == L.MLA_ERR_NULL
    assert call(o_lat=FAKE + 4) == L.MLA_ERR_UNSUPPORTED
    assert call(B=0) == L.MLA_OK


def test_partial_warm_validation(lib):
    f = lib.mla_decode_partial_warm
    d = _desc()
    need = lib.mla_decode_workspace_bytes(1, 128, 512, 4096, 0)

    def call(warm=FAKE, nbytes=1 << 20, ws=FAKE, B=1):
        return f(FAKE, FAKE, L.MLA_BF16, ctypes.byref(d), FAKE, 4096, B, 128, 512, 64, 1 / math.sqrt(192), 0, ws, need,
                 warm, nbytes, None)
    assert call(ws=None) == L.MLA_ERR_WORKSPACE
    assert call(warm=None) == L.MLA_ERR_NULL
    assert call(warm=FAKE + 2) == L.MLA_ERR_UNSUPPORTED
    assert call(B=0) == L.MLA_OK


def test_cache_append_validation(lib):
    f = lib.mla_cache_append
    ws = lib.mla_cache_append_workspace_bytes
    # the two-pass form's 14 chunk partials (the one-pass bf16 form up to 8 tokens needs none)
    assert ws(1, 7168) == 14 * 1 * 576 * 4 and ws(128, 7168) == 14 * 128 * 576 * 4
    assert ws(0, 7168) == 0 and ws(1, 7000) == 0 and ws(1, 0) == 0
    good_ws = ws(4, 7168)

    def call(desc, B=4, D=7168, d_c=512, d_R=64, base=10000.0, dtype=L.MLA_BF16, h=FAKE, wsp=FAKE, wsb=good_ws,
             pos=FAKE):
        return f(h, FAKE, FAKE, dtype, pos, ctypes.byref(desc), B, D, d_c, d_R, base, wsp, wsb, None)

    d = _desc()
    assert call(d, B=-1) == L.MLA_ERR_SHAPE
    assert call(d, base=0.0) == L.MLA_ERR_SHAPE
    assert call(d, base=math.inf) == L.MLA_ERR_SHAPE
    assert call(d, dtype=7) == L.MLA_ERR_DTYPE
    assert call(d, B=0, h=None, pos=None) == L.MLA_OK                   # no-op
    assert call(d, pos=None) == L.MLA_ERR_NULL
    assert f(FAKE, FAKE, FAKE, L.MLA_BF16, FAKE, None, 4, 7168, 512, 64, 1e4, FAKE, good_ws, None) == L.MLA_ERR_NULL
    assert call(d, dtype=L.MLA_F32) == L.MLA_ERR_UNSUPPORTED
    assert call(d, d_c=256) == L.MLA_ERR_UNSUPPORTED
    assert call(d, d_R=32) == L.MLA_ERR_UNSUPPORTED
    assert call(d, D=7000) == L.MLA_ERR_UNSUPPORTED
    assert call(d, h=FAKE + 2) == L.MLA_ERR_UNSUPPORTED
    assert call(d, wsp=None) == L.MLA_ERR_WORKSPACE
    assert call(d, wsb=good_ws - 1) == L.MLA_ERR_WORKSPACE
    assert call(d, wsp=FAKE + 4) == L.MLA_ERR_UNSUPPORTED
    assert call(_desc(latent_dtype=L.MLA_F32)) == L.MLA_ERR_UNSUPPORTED
    assert call(_desc(latent_dtype=L.MLA_FP8_E4M3)) == L.MLA_ERR_NULL     # fp8 needs the scale
    assert call(_desc(st_tok=577)) == L.MLA_ERR_UNSUPPORTED               # unaligned rows
    assert call(_desc(bt=FAKE, page=0, max_pages=4)) == L.MLA_ERR_SHAPE   # paged without a page size


def test_mha_decode_validation(lib):
    f = lib.mla_mha_decode
    ws = lib.mla_mha_decode_workspace_bytes
    assert ws(1, 128, 4096, 0) == 1 * 128 * 8 * 130 * 4     # auto: min(32, ceil(1024/128)) = 8 splits
    assert ws(2, 8, 300, 3) == 2 * 8 * 3 * 130 * 4 and ws(0, 8, 300, 3) == 0

    def call(B=2, H=8, d_k=192, d_v=128, max_len=300, cap=320, dtype=L.MLA_BF16, scale=0.07, splits=3, wsp=FAKE,
             wsb=1 << 30, q=FAKE, out=FAKE):
        return f(q, FAKE, FAKE, dtype, FAKE, max_len, cap, B, H, d_k, d_v, scale, splits, wsp, wsb, out, None, None)

    assert call(B=-1) == L.MLA_ERR_SHAPE
    assert call(cap=0) == L.MLA_ERR_SHAPE
    assert call(max_len=321) == L.MLA_ERR_SHAPE             # longer than the cache
    assert call(scale=-1.0) == L.MLA_ERR_SHAPE
    assert call(dtype=5) == L.MLA_ERR_DTYPE
    assert call(B=0, q=None, out=None) == L.MLA_OK
    assert call(out=None) == L.MLA_ERR_NULL
    assert call(d_k=128) == L.MLA_ERR_UNSUPPORTED
    assert call(dtype=L.MLA_F32) == L.MLA_ERR_UNSUPPORTED
    assert call(q=FAKE + 8) == L.MLA_ERR_UNSUPPORTED
    assert call(wsb=100) == L.MLA_ERR_WORKSPACE


def test_projection_workspace_rules(lib):
    ws = lib.mla_proj_workspace_bytes
    # GEMV (no workspace): up to 4 tokens, or up to 8 with K >= 4096 and at most 32M weight elements
    assert ws(1, 1536, 7168) == 0 and ws(4, 7168, 16384) == 0 and ws(4, 24576, 1536) == 0
    assert ws(8, 1536, 7168) == 0 and ws(8, 2112, 7168) == 0 and ws(8, 576, 7168) == 0
    assert ws(8, 7168, 16384) == 4 * 8 * 7168 * 4                            # W_O at 5-8 tokens: MFMA
    assert ws(5, 24576, 1536) == 2 * 5 * 24576 * 4                            # K < 4096: MFMA path
    # MFMA path: tiles of 128 rows x 128 tokens; K split into d chunks, d the smallest divisor of
    # K / 256 that gives at least 224 workgroups and chunks of at most 4096 elements (else K / 256)
    assert ws(9, 1536, 7168) == 28 * 9 * 1536 * 4                             # 12 tiles: 28 chunks
    assert ws(9, 2112, 7168) == 14 * 9 * 2112 * 4                             # 17 tiles: 14 chunks
    assert ws(64, 24576, 1536) == 2 * 64 * 24576 * 4                          # 192 tiles: 2 chunks
    assert ws(128, 7168, 16384) == 4 * 128 * 7168 * 4                         # 56 tiles: 4 chunks
    assert ws(129, 7168, 16384) == 4 * 129 * 7168 * 4                         # 112 tiles: 4 chunks (<= 4096)
    assert ws(64, 7168, 65536) == 16 * 64 * 7168 * 4                          # folded W_OV: 16 chunks
    assert ws(0, 32, 512) == 0
    q = lib.mla_query_workspace_bytes
    assert q(1, 7168, 1536, 128, 128, 64) == 0 and q(2, 7168, 1536, 128, 128, 64) == 0
    assert q(8, 7168, 1536, 128, 128, 64) == ws(8, 128 * 192, 1536) > 0     # second pass on MFMA
    assert q(64, 7168, 1536, 128, 128, 64) == max(ws(64, 1536, 7168), ws(64, 128 * 192, 1536))


def test_query_proj_validation(lib):
    f = lib.mla_query_proj

    def call(B=1, D=7168, d_q=1536, H=128, d_h=128, d_R=64, base=1e4, dtype=L.MLA_BF16, h=FAKE, pos=FAKE,
             out=FAKE, wsp=None, wsb=0):
        return f(h, FAKE, FAKE, FAKE, dtype, pos, B, D, d_q, H, d_h, d_R, base, out, FAKE, FAKE, wsp, wsb, None)

    assert call(B=-1) == L.MLA_ERR_SHAPE
    assert call(base=-1.0) == L.MLA_ERR_SHAPE
    assert call(dtype=9) == L.MLA_ERR_DTYPE
    assert call(B=0, h=None, pos=None) == L.MLA_OK
    assert call(pos=None) == L.MLA_ERR_NULL
    assert call(out=None) == L.MLA_ERR_NULL
    assert call(dtype=L.MLA_F32) == L.MLA_ERR_UNSUPPORTED
    assert call(d_R=32) == L.MLA_ERR_UNSUPPORTED
    assert call(D=7000) == L.MLA_ERR_UNSUPPORTED
    assert call(d_q=1000) == L.MLA_ERR_UNSUPPORTED
    assert call(h=FAKE + 2) == L.MLA_ERR_UNSUPPORTED
    assert call(H=3, d_h=6) == L.MLA_ERR_UNSUPPORTED                      # q_C rows not a multiple of 8
    need = lib.mla_query_workspace_bytes(64, 7168, 1536, 128, 128, 64)
    assert call(B=64) == L.MLA_ERR_WORKSPACE
    assert call(B=64, wsp=FAKE, wsb=need - 1) == L.MLA_ERR_WORKSPACE
    assert call(B=64, wsp=FAKE + 8, wsb=need) == L.MLA_ERR_UNSUPPORTED


def test_fold_and_out_proj_validation(lib):
    fq, fo, ab, op = lib.mla_fold_q, lib.mla_fold_o, lib.mla_absorb_q_folded, lib.mla_out_proj
    assert fq(FAKE, FAKE, L.MLA_BF16, FAKE, 0, 128, 512, 1536, None) == L.MLA_ERR_SHAPE
    assert fq(FAKE, FAKE, 7, FAKE, 128, 128, 512, 1536, None) == L.MLA_ERR_DTYPE
    assert fq(None, FAKE, L.MLA_BF16, FAKE, 128, 128, 512, 1536, None) == L.MLA_ERR_NULL
    assert fq(FAKE, FAKE, L.MLA_F32, FAKE, 128, 128, 512, 1536, None) == L.MLA_ERR_UNSUPPORTED
    assert fq(FAKE, FAKE, L.MLA_BF16, FAKE, 128, 100, 512, 1536, None) == L.MLA_ERR_UNSUPPORTED
    assert fo(FAKE, FAKE, L.MLA_BF16, FAKE, 7000, 128, 128, 512, None) == L.MLA_ERR_UNSUPPORTED
    assert fo(FAKE, FAKE, L.MLA_BF16, None, 7168, 128, 128, 512, None) == L.MLA_ERR_NULL
    assert ab(FAKE, FAKE, L.MLA_BF16, FAKE, L.MLA_BF16, 0, 128, 512, 1536, None, 0, None) == L.MLA_OK
    assert ab(FAKE, FAKE, L.MLA_BF16, FAKE, L.MLA_FP8_E4M3, 1, 128, 512, 1536, None, 0, None) == L.MLA_ERR_UNSUPPORTED
    assert ab(FAKE, FAKE, L.MLA_BF16, FAKE, L.MLA_BF16, 1, 128, 512, 1000, None, 0, None) == L.MLA_ERR_UNSUPPORTED
    assert ab(FAKE, FAKE, L.MLA_BF16, FAKE, L.MLA_BF16, 16, 128, 512, 1536, None, 0, None) == L.MLA_ERR_WORKSPACE
    assert op(FAKE, FAKE, L.MLA_BF16, FAKE, -1, 7168, 16384, None, 0, None) == L.MLA_ERR_SHAPE
    assert op(FAKE, FAKE, L.MLA_F32, FAKE, 1, 7168, 16384, None, 0, None) == L.MLA_ERR_UNSUPPORTED
    assert op(FAKE, FAKE, L.MLA_BF16, FAKE, 1, 7000, 16384, None, 0, None) == L.MLA_ERR_UNSUPPORTED
    assert op(FAKE, FAKE, L.MLA_BF16, FAKE, 1, 7168, 16000, None, 0, None) == L.MLA_ERR_UNSUPPORTED
    assert op(FAKE + 4, FAKE, L.MLA_BF16, FAKE, 1, 7168, 16384, None, 0, None) == L.MLA_ERR_UNSUPPORTED
    assert op(FAKE, FAKE, L.MLA_BF16, FAKE, 9, 7168, 16384, None, 0, None) == L.MLA_ERR_WORKSPACE
    assert op(FAKE, FAKE, L.MLA_BF16, FAKE, 16384, 7168, 65536, FAKE, 1 << 40, None) == L.MLA_ERR_UNSUPPORTED


def test_query_proj_append_validation(lib):
    f = lib.mla_query_proj_append
    ws = lib.mla_query_append_workspace_bytes
    assert ws(1, 7168, 1536, 128, 128, 64, 512) == 0                          # GEMV passes
    assert ws(64, 7168, 1536, 128, 128, 64, 512) == max(
        lib.mla_proj_workspace_bytes(64, 1536 + 576, 7168), lib.mla_proj_workspace_bytes(64, 128 * 192, 1536))

    def call(desc, B=1, dtype=L.MLA_BF16, d_c=512, d_R=64, pos=FAKE, wsp=None, wsb=0):
        return f(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, dtype, pos, ctypes.byref(desc), B, 7168, 1536, 128, 128, d_R, d_c,
                 1e4, FAKE, FAKE, FAKE, wsp, wsb, None)

    d = _desc()
    assert call(d, B=-1) == L.MLA_ERR_SHAPE
    assert call(d, dtype=7) == L.MLA_ERR_DTYPE
    assert call(d, B=0, pos=None) == L.MLA_OK
    assert call(d, pos=None) == L.MLA_ERR_NULL
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, L.MLA_BF16, FAKE, None, 1, 7168, 1536, 128, 128, 64, 512, 1e4, FAKE,
             FAKE, FAKE, None, 0, None) == L.MLA_ERR_NULL
    assert call(_desc(latent_dtype=L.MLA_FP8_E4M3)) == L.MLA_ERR_UNSUPPORTED   # E4M3: the two separate calls
    assert call(d, d_c=256) == L.MLA_ERR_UNSUPPORTED
    assert call(_desc(st_tok=577)) == L.MLA_ERR_UNSUPPORTED
    assert call(d, B=64) == L.MLA_ERR_WORKSPACE
