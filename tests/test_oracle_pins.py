"""Pins of the CPU oracle against facts fixed by the pages and by mathematics.

Each test ties one part of the oracle to something other than itself: the
worked example's printed keys and values, printed cache-size figures, closed
forms of softmax attention, torch's scaled_dot_product_attention on the CPU,
and the absorption identities.  ``test_planted_mistakes_are_caught`` plants
plausible mistakes in the oracle and checks that these pins catch each one.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np
import pytest

import oracle
from oracle import cache_size as cs
import oracle.mla_decode as od
from oracle.mla_decode import merge_partials
from tests._helpers import custom_inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# --------------------------------------------------------------------------
# worked example ("MLA storage: Representing KV with a small latent vector")
# --------------------------------------------------------------------------
def _worked_weights(g):
    # the page's projections are row-vector [d_c x d_h]; the oracle takes W[h] = U^T ([d_h x d_c])
    W_UK = np.stack([np.array(g["U1K_rowvector_3x2"]).T, np.array(g["U2K_rowvector_3x2_reconstructed"]).T])
    W_UV = np.stack([np.array(g["U1V_rowvector_3x2_reconstructed"]).T, np.array(g["U2V_rowvector_3x2_reconstructed"]).T])
    return W_UK.astype(np.float64), W_UV.astype(np.float64)


def check_worked_example_kv():
    g = _golden("worked_example.json")
    W_UK, W_UV = _worked_weights(g)
    c = np.array([g["latent_c3"]], dtype=np.float64)
    r = np.array([[0.25, -0.5]])
    for h, name in enumerate(["head1", "head2"]):
        K, V = od.expand_kv(c, r, W_UK[h], W_UV[h])
        exp_k = g["expected_content_key"][name] + [0.25, -0.5]
        np.testing.assert_array_equal(K[0], exp_k)
        np.testing.assert_array_equal(V[0], g["expected_value"][name])


def test_worked_example_keys_and_values():
    check_worked_example_kv()


def check_worked_example_one_token_output():
    """With one cached token the softmax weight is 1, so the output is that token's value."""
    g = _golden("worked_example.json")
    W_UK, W_UV = _worked_weights(g)
    rng = np.random.default_rng(0)
    inp = custom_inputs(q_C=rng.standard_normal((1, 2, 2)), q_R=rng.standard_normal((1, 2, 2)),
                        W_UK=W_UK, W_UV=W_UV, C_rows=[np.array([g["latent_c3"]])],
                        R_rows=[np.array([[0.25, -0.5]])])
    out = od.decode(inp)
    np.testing.assert_allclose(out["o"][0, 0], g["expected_value"]["head1"], rtol=0, atol=1e-12)
    np.testing.assert_allclose(out["o"][0, 1], g["expected_value"]["head2"], rtol=0, atol=1e-12)


def test_worked_example_single_token_output():
    check_worked_example_one_token_output()


def test_worked_example_cache_growth():
    g = _golden("worked_example.json")
    per = cs.mla_values(d_c=3, d_R=2)
    assert per == g["stored_components_per_token"]
    assert cs.stored_components(4, per) == g["stored_components_4_tokens"]
    assert cs.stored_components(5, per) == g["stored_components_5_tokens"]
    m = g["toy_mha"]
    assert cs.mha_values(m["kv_heads"], m["head_dim"]) == m["per_token"]
    assert cs.stored_components(4, m["per_token"]) == m["4_tokens"]
    assert cs.stored_components(5, m["per_token"]) == m["5_tokens"]
    q = g["toy_gqa"]
    assert cs.gqa_values(q["kv_heads"], q["head_dim"]) == q["per_token"]
    assert cs.stored_components(4, q["per_token"]) == q["4_tokens"]
    assert cs.stored_components(5, q["per_token"]) == q["5_tokens"]


# --------------------------------------------------------------------------
# cache-size figures printed on the pages
# --------------------------------------------------------------------------
def test_cache_size_dimensional_example():
    g = _golden("cache_sizes.json")["dimensional_example"]
    vals = {"MHA": cs.mha_values(g["heads"], g["head_dim"]),
            "GQA": cs.gqa_values(g["gqa_groups"], g["head_dim"]),
            "MQA": cs.mqa_values(g["head_dim"]),
            "MLA": cs.mla_values(g["mla_latent"], g["mla_rope"])}
    assert vals == g["values_per_token_layer"]
    for k, pct in g["relative_to_mha_percent"].items():
        assert round(100.0 * vals[k] / vals["MHA"], 3 if k == "MQA" else 2) == pct
    assert cs.cache_bytes(vals["MHA"], g["layers"], g["context"], 1, g["bytes_per_value"]) == g["mha_sequence_bytes"]
    for k, gib in g["gib"].items():
        assert round(cs.cache_gib(vals[k], g["layers"], g["context"], 1, g["bytes_per_value"]), 3) == pytest.approx(gib, abs=1e-9)
    assert round(vals["MHA"] / vals["MLA"], 1) == g["mla_smaller_factor"]


def test_cache_size_v3_and_57x_and_70b():
    g = _golden("cache_sizes.json")
    v3 = g["v3"]
    assert cs.mla_values(v3["d_c"], v3["d_R"]) == v3["mla_values"]
    # plain multi-head with the same head sizes: keys 128+64 wide, values 128 wide, per head
    assert v3["heads"] * ((v3["content_head_dim"] + v3["d_R"]) + v3["content_head_dim"]) == v3["plain_mha_same_head_sizes"]
    assert cs.mla_values(v3["d_c"], v3["d_R"]) / v3["content_head_dim"] == v3["mla_over_head_dim"]
    v2 = g["v2_57x"]
    factor = cs.mha_values(v2["heads"], v2["head_dim"]) / cs.mla_values(v2["d_c"], v2["d_R"])
    assert round(factor) == v2["headline_factor"]
    ll = g["llama2_70b"]
    b = cs.cache_bytes(cs.mha_values(ll["heads"], ll["head_dim"]), ll["layers"], ll["tokens"], ll["batch"], ll["bytes_per_value"])
    assert round(b / 1e9) == ll["gigabytes"]


# --------------------------------------------------------------------------
# closed forms
# --------------------------------------------------------------------------
def _tiny_two_dim(C, R, qC, qR):
    """d_c=2, d_h=1, d_R=1: key content = first latent component, value = second."""
    W_UK = np.array([[[1.0, 0.0]]])
    W_UV = np.array([[[0.0, 1.0]]])
    return custom_inputs(q_C=[[[qC]]], q_R=[[[qR]]], W_UK=W_UK, W_UV=W_UV,
                         C_rows=[np.asarray(C, dtype=np.float64)], R_rows=[np.asarray(R, dtype=np.float64)])


def check_two_token_sigmoid():
    C = [[0.5, 3.0], [-1.0, -2.0]]
    R = [[0.25], [1.5]]
    qC, qR = 2.0, -1.0
    inp = _tiny_two_dim(C, R, qC, qR)
    out = od.decode(inp)
    sc = 1.0 / math.sqrt(2.0)
    s0 = (qC * 0.5 + qR * 0.25) * sc
    s1 = (qC * -1.0 + qR * 1.5) * sc
    a1 = 1.0 / (1.0 + math.exp(-(s1 - s0)))
    expect = (1 - a1) * 3.0 + a1 * -2.0
    assert out["o"][0, 0, 0] == pytest.approx(expect, rel=1e-14, abs=1e-14)
    assert out["lse"][0, 0] == pytest.approx(math.log(math.exp(s0) + math.exp(s1)), rel=1e-14)


def test_two_tokens_weight_is_sigmoid_of_score_gap():
    check_two_token_sigmoid()


def check_zero_query_uniform():
    rng = np.random.default_rng(1)
    H, d_h, d_c, d_R, L = 3, 4, 6, 2, 7
    W_UK = rng.standard_normal((H, d_h, d_c))
    W_UV = rng.standard_normal((H, d_h, d_c))
    C = rng.standard_normal((L, d_c))
    R = rng.standard_normal((L, d_R))
    inp = custom_inputs(q_C=np.zeros((1, H, d_h)), q_R=np.zeros((1, H, d_R)), W_UK=W_UK, W_UV=W_UV,
                        C_rows=[C], R_rows=[R])
    out = od.decode(inp)
    Cf = C.astype(np.float32).astype(np.float64)
    for h in range(H):
        expect = W_UV[h].astype(np.float32).astype(np.float64) @ Cf.mean(axis=0)
        np.testing.assert_allclose(out["o"][0, h], expect, rtol=1e-12, atol=1e-12)
        assert out["lse"][0, h] == pytest.approx(math.log(L), rel=1e-14)


def test_zero_query_gives_uniform_weights():
    check_zero_query_uniform()


def test_empty_sequence_gives_zero_output():
    rng = np.random.default_rng(2)
    inp = custom_inputs(q_C=rng.standard_normal((2, 2, 4)), q_R=rng.standard_normal((2, 2, 2)),
                        W_UK=rng.standard_normal((2, 4, 8)), W_UV=rng.standard_normal((2, 4, 8)),
                        C_rows=[np.zeros((0, 8)), rng.standard_normal((3, 8))],
                        R_rows=[np.zeros((0, 2)), rng.standard_normal((3, 2))], n_max=4)
    out = od.decode(inp)
    assert np.all(out["o"][0] == 0.0) and np.all(out["o_lat"][0] == 0.0)
    assert np.all(np.isneginf(out["lse"][0]))
    assert np.all(np.isfinite(out["o"][1]))


# --------------------------------------------------------------------------
# library special case: torch scaled_dot_product_attention on explicit K/V
# --------------------------------------------------------------------------
def check_against_sdpa(seed=3):
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(seed)
    B, H, d_h, d_c, d_R = 3, 5, 8, 16, 4
    lens = [1, 6, 11]
    W_UK = rng.standard_normal((H, d_h, d_c)) / 4
    W_UV = rng.standard_normal((H, d_h, d_c)) / 4
    q_C = rng.standard_normal((B, H, d_h))
    q_R = rng.standard_normal((B, H, d_R))
    C = [rng.standard_normal((L, d_c)) for L in lens]
    R = [rng.standard_normal((L, d_R)) for L in lens]
    inp = custom_inputs(q_C, q_R, W_UK, W_UV, C, R)
    out = od.decode(inp)
    f = lambda a: torch.tensor(np.asarray(a, dtype=np.float32).astype(np.float64))  # noqa: E731
    N = max(lens)
    for b in range(B):
        L = lens[b]
        Cb = torch.zeros(N, d_c, dtype=torch.float64)
        Rb = torch.zeros(N, d_R, dtype=torch.float64)
        Cb[:L] = f(C[b])
        Rb[:L] = f(R[b])
        Wk, Wv = f(W_UK), f(W_UV)
        K = torch.cat([torch.einsum("nc,hdc->hnd", Cb, Wk), Rb.expand(H, N, d_R)], dim=-1)
        V = torch.einsum("nc,hdc->hnd", Cb, Wv)
        Q = torch.cat([f(q_C[b]), f(q_R[b])], dim=-1)[:, None, :]
        mask = torch.zeros(H, 1, N, dtype=torch.bool)
        mask[..., :L] = True
        ref = torch.nn.functional.scaled_dot_product_attention(Q[None], K[None], V[None], attn_mask=mask[None])
        np.testing.assert_allclose(out["o"][b], ref[0, :, 0].numpy(), rtol=1e-10, atol=1e-12)


def test_oracle_matches_torch_sdpa():
    check_against_sdpa()


# --------------------------------------------------------------------------
# absorption identities ("Grouped-query and latent attention", "The absorption trick")
# --------------------------------------------------------------------------
def check_absorption(seed=4):
    rng = np.random.default_rng(seed)
    B, H, d_h, d_c, d_R = 2, 4, 8, 24, 6
    lens = [9, 17]
    W_UK = rng.standard_normal((H, d_h, d_c)) / 5
    W_UV = rng.standard_normal((H, d_h, d_c)) / 5
    q_C = rng.standard_normal((B, H, d_h))
    q_R = rng.standard_normal((B, H, d_R))
    C = [rng.standard_normal((L, d_c)) for L in lens]
    R = [rng.standard_normal((L, d_R)) for L in lens]
    inp = custom_inputs(q_C, q_R, W_UK, W_UV, C, R)
    out = od.decode(inp)
    sc = 1.0 / math.sqrt(d_h + d_R)
    for b in range(B):
        Cb = np.asarray(C[b], dtype=np.float32).astype(np.float64)
        Rb = np.asarray(R[b], dtype=np.float32).astype(np.float64)
        qR = q_R[b].astype(np.float32).astype(np.float64)
        for h in range(H):
            # folded query against the latents plus the rope term: the same log-sum-exp
            s_abs = (Cb @ out["q_abs"][b, h] + Rb @ qR[h]) * sc
            lse = np.max(s_abs) + np.log(np.sum(np.exp(s_abs - np.max(s_abs))))
            assert abs(lse - out["lse"][b, h]) <= 1e-12 * max(1.0, abs(lse))
            # value side: W_UV applied once to the weighted latent sum
            o2 = W_UV[h].astype(np.float32).astype(np.float64) @ out["o_lat"][b, h]
            np.testing.assert_allclose(o2, out["o"][b, h], rtol=1e-12, atol=1e-13)


def test_absorption_identities_hold_for_oracle_diagnostics():
    check_absorption()


def test_oracle_float32_agrees_with_float64():
    from workloads import make_inputs
    inp = make_inputs(1)
    o64 = od.decode(inp, dtype=np.float64)["o"]
    o32 = od.decode(inp, dtype=np.float32)["o"]
    assert oracle.relative_l2(o32, o64) <= 1e-6


# --------------------------------------------------------------------------
# split-N merge definition
# --------------------------------------------------------------------------
def test_merge_partials_equals_one_pass():
    rng = np.random.default_rng(5)
    L, d = 37, 5
    s = rng.standard_normal(L) * 3
    x = rng.standard_normal((L, d))
    a = np.exp(s - s.max())
    ref = (a / a.sum()) @ x
    ref_lse = s.max() + np.log(a.sum())
    for cuts in ([0, L], [0, 1, L], [0, 5, 5, 20, L], [0, 13, 26, 36, L], list(range(L + 1))):
        ms, ls, accs = [], [], []
        for lo, hi in zip(cuts[:-1], cuts[1:]):
            if hi == lo:
                ms.append(-np.inf); ls.append(0.0); accs.append(np.zeros(d))
                continue
            m = s[lo:hi].max()
            e = np.exp(s[lo:hi] - m)
            ms.append(m); ls.append(e.sum()); accs.append(e @ x[lo:hi])
        out, lse = merge_partials(ms, ls, accs)
        np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-14)
        assert lse == pytest.approx(ref_lse, rel=1e-13)
    out, lse = merge_partials([-np.inf, -np.inf], [0.0, 0.0], [np.zeros(d), np.zeros(d)])
    assert np.all(out == 0) and lse == -np.inf


# --------------------------------------------------------------------------
# storage decoders
# --------------------------------------------------------------------------
def test_e4m3_decoder_special_values():
    # OCP 8-bit floating point specification, E4M3 column: bias 7, no infinities,
    # S.1111.111 = NaN, max normal S.1111.110 = 448, min normal 2^-6, min subnormal 2^-9
    d = oracle.decode_e4m3
    assert d(0x00) == 0.0 and np.signbit(d(0x80)) and d(0x80) == 0.0
    assert d(0x7E) == 448.0 and d(0xFE) == -448.0
    assert d(0x08) == 2.0 ** -6
    assert d(0x01) == 2.0 ** -9 and d(0x07) == 7 * 2.0 ** -9
    assert d(0x38) == 1.0 and d(0x3C) == 1.5 and d(0xC0) == -2.0
    assert np.isnan(d(0x7F)) and np.isnan(d(0xFF))
    assert d(0x78) == 256.0 and d(0x77) == 240.0
    vals = oracle.decode_e4m3(np.arange(256, dtype=np.uint8))
    assert np.isnan(vals).sum() == 2
    pos = vals[:0x7F]
    assert np.all(np.diff(pos) > 0)  # codes 0..0x7E are strictly increasing


def test_bf16_decoder_values():
    d = oracle.decode_bf16
    assert d(0x3F80) == 1.0 and d(0xC000) == -2.0 and d(0x0000) == 0.0
    assert np.isinf(d(0x7F80)) and np.isnan(d(0x7FC0))
    assert d(0x3F81) == 1.0 + 2.0 ** -7
    assert d(0x0001) == 2.0 ** -133


# --------------------------------------------------------------------------
# planted mistakes: each must fail at least one of the pins above
# --------------------------------------------------------------------------
_attend = od.attend

PIN_CHECKS = [check_worked_example_kv, check_worked_example_one_token_output, check_two_token_sigmoid,
              check_zero_query_uniform, check_against_sdpa, check_absorption]


def _mut_expand_kv_rope_added(C_b, R_b, W_UK_h, W_UV_h):
    K_C = C_b @ W_UK_h.T
    K = np.concatenate([K_C, np.zeros_like(R_b)], axis=1)   # rope term dropped
    return K, C_b @ W_UV_h.T


def _mut_expand_kv_value_uses_key_proj(C_b, R_b, W_UK_h, W_UV_h):
    K_C = C_b @ W_UK_h.T
    return np.concatenate([K_C, R_b], axis=1), C_b @ W_UK_h.T


def _mut_expand_kv_rope_into_value(C_b, R_b, W_UK_h, W_UV_h):
    K = np.concatenate([C_b @ W_UK_h.T, R_b], axis=1)
    V = C_b @ W_UV_h.T
    V = V + np.resize(R_b.sum(axis=1, keepdims=True), V.shape)
    return K, V


def _mut_attend_wrong_scale(K, V, q, scale):
    return _attend(K, V, q, 1.0 / math.sqrt(K.shape[1] - 1))


def _mut_attend_no_softmax_norm(K, V, q, scale):
    o, lse, a = _attend(K, V, q, scale)
    if K.shape[0] == 0:
        return o, lse, a
    s = (K @ q) * scale
    e = np.exp(s - s.max())
    return e @ V, lse, e


def _mut_attend_drops_last_token(K, V, q, scale):
    if K.shape[0] > 1:
        return _attend(K[:-1], V[:-1], q, scale)
    return _attend(K, V, q, scale)


MUTANTS = {
    "rope_term_dropped": ("expand_kv", _mut_expand_kv_rope_added),
    "value_uses_W_UK": ("expand_kv", _mut_expand_kv_value_uses_key_proj),
    "rope_leaks_into_value": ("expand_kv", _mut_expand_kv_rope_into_value),
    "scale_off_by_one_dim": ("attend", _mut_attend_wrong_scale),
    "softmax_not_normalised": ("attend", _mut_attend_no_softmax_norm),
    "last_token_skipped": ("attend", _mut_attend_drops_last_token),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistakes_are_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(od, attr, fn)
    failures = 0
    for chk in PIN_CHECKS:
        try:
            chk()
        except (AssertionError, ValueError):
            failures += 1
    assert failures >= 1, f"planted mistake {name!r} passed every pin"


# --------------------------------------------------------------------------
# the error metric and the cache read, pinned by hand-computed cases
# --------------------------------------------------------------------------
def check_relative_l2_hand_cases():
    """||x - ref||_2 / ||ref||_2, worked by hand."""
    rl2 = od.relative_l2
    # diff (0, 2, 2): norm sqrt(8); ref norm 1
    assert rl2([1.0, 2.0, 2.0], [1.0, 0.0, 0.0]) == pytest.approx(math.sqrt(8.0), rel=1e-15)
    # diff (0.1, 0): 0.1 / sqrt(2) -- a norm ratio, not the largest elementwise error (0.1)
    assert rl2([1.1, 1.0], [1.0, 1.0]) == pytest.approx(0.1 / math.sqrt(2.0), rel=1e-12)
    # diff (3, 4) over ref (6, 8): 5 / 10
    assert rl2([9.0, 12.0], [6.0, 8.0]) == pytest.approx(0.5, rel=1e-15)
    # NaN entries of the reference (pairs not computed) are skipped: diff (1, 0) over ref (1, 0)
    assert rl2([2.0, 100.0, 0.0], [1.0, np.nan, 0.0]) == pytest.approx(1.0, rel=1e-15)
    # a zero reference gives the absolute norm of x
    assert rl2([3.0, 4.0], [0.0, 0.0]) == pytest.approx(5.0, rel=1e-15)
    # identical arrays: exactly zero; 2-D arrays are flattened
    assert rl2(np.ones((2, 3)), np.ones((2, 3))) == 0.0
    assert rl2([[1.0, 0.0], [0.0, 0.0]], [[0.0, 0.0], [0.0, 2.0]]) == pytest.approx(math.sqrt(5.0) / 2.0, rel=1e-15)


def test_relative_l2_hand_cases():
    check_relative_l2_hand_cases()


def _bf16_bits(vals):
    """Bit patterns of values exactly representable in bfloat16 (small integers here), written
    out from the float32 bit pattern; NaN -> 0x7FC0."""
    out = []
    for v in np.asarray(vals, dtype=np.float64).reshape(-1):
        if math.isnan(v):
            out.append(0x7FC0)
        else:
            u = int(np.array([v], dtype=np.float32).view(np.uint32)[0])
            assert u & 0xFFFF == 0, v
            out.append(u >> 16)
    return np.array(out, dtype=np.uint16).reshape(np.shape(vals))


def _tiny_wl(layout, B, n_max, dtype="bf16", page_size=64):
    from workloads.configs import Workload
    return Workload("hand", seed=0, B=B, H=1, d_h=1, d_c=2, d_R=1, n_max=n_max, len_lo=0, len_hi=n_max,
                    dtype=dtype, layout=layout, page_size=page_size)


def check_gather_rows_hand_placed():
    """Rows placed by hand in each cache layout; latent columns first, then the rope columns
    ("MLA storage: Representing KV with a small latent vector", section "Storing a positional key
    separately": a cached row is the latent followed by the rope key).  d_c = 2, d_R = 1."""
    from workloads.gen import DecodeInputs
    nan = float("nan")
    z = np.zeros((2, 1, 1), dtype=np.uint16)
    # packed [B=2, n_max=3, 3]: sequence 0 holds two tokens, sequence 1 three
    kv = _bf16_bits([[[1, 2, 3], [4, 5, 6], [nan, nan, nan]],
                     [[7, 8, 9], [10, 11, 12], [13, 14, 15]]])
    pk = DecodeInputs(wl=_tiny_wl("packed", 2, 3), lens=np.array([2, 3], dtype=np.int32),
                      q_C=z, q_R=z, W_UK=z, W_UV=z, kv=kv)
    C, R = od.gather_rows(pk, 0)
    np.testing.assert_array_equal(C, [[1, 2], [4, 5]])
    np.testing.assert_array_equal(R, [[3], [6]])
    C, R = od.gather_rows(pk, 1)
    np.testing.assert_array_equal(C, [[7, 8], [10, 11], [13, 14]])
    np.testing.assert_array_equal(R, [[9], [12], [15]])
    # paged: pages of 2 tokens, block table [[3, 1], [0, 2]]; sequence 0 has 3 tokens (page 3
    # slots 0, 1, then page 1 slot 0), sequence 1 has 2 (page 0 slots 0, 1); the rest is padding
    pool = np.full((4, 2, 3), nan)
    pool[3, 0] = [1, 2, 3]
    pool[3, 1] = [4, 5, 6]
    pool[1, 0] = [7, 8, 9]
    pool[0, 0] = [10, 11, 12]
    pool[0, 1] = [13, 14, 15]
    pg = DecodeInputs(wl=_tiny_wl("paged", 2, 4, page_size=2), lens=np.array([3, 2], dtype=np.int32),
                      q_C=z, q_R=z, W_UK=z, W_UV=z, pool=_bf16_bits(pool),
                      block_table=np.array([[3, 1], [0, 2]], dtype=np.int32))
    C, R = od.gather_rows(pg, 0)
    np.testing.assert_array_equal(C, [[1, 2], [4, 5], [7, 8]])
    np.testing.assert_array_equal(R, [[3], [6], [9]])
    C, R = od.gather_rows(pg, 1)
    np.testing.assert_array_equal(C, [[10, 11], [13, 14]])
    np.testing.assert_array_equal(R, [[12], [15]])
    # split fp8: E4M3 codes 0x38 = 1.0, 0x40 = 2.0, 0x30 = 0.5, 0xB8 = -1.0, times the token's scale
    lat = np.array([[[0x38, 0x40], [0x30, 0xB8], [0x7F, 0x7F]]], dtype=np.uint8)
    scale = np.array([[2.0, 0.25, nan]], dtype=np.float32)
    rope = _bf16_bits([[[3], [-6], [nan]]])
    f8 = DecodeInputs(wl=_tiny_wl("split", 1, 3, dtype="fp8"), lens=np.array([2], dtype=np.int32),
                      q_C=z, q_R=z, W_UK=z, W_UV=z, latent=lat, rope=rope, scale=scale)
    C, R = od.gather_rows(f8, 0)
    np.testing.assert_array_equal(C, [[2.0, 4.0], [0.125, -0.25]])
    np.testing.assert_array_equal(R, [[3], [-6]])


def test_gather_rows_hand_placed():
    check_gather_rows_hand_placed()


_gather = od.gather_rows


def _mut_gather_packed_columns_swapped(inp, b):
    if inp.wl.layout != "packed":
        return _gather(inp, b)
    rows = od.decode_bf16(inp.kv[b, :int(inp.lens[b])])
    return rows[:, inp.wl.d_R:], rows[:, :inp.wl.d_R]


def _mut_gather_paged_index_transposed(inp, b):
    if inp.wl.layout != "paged":
        return _gather(inp, b)
    P, L, d_c = inp.wl.page_size, int(inp.lens[b]), inp.wl.d_c
    j = np.arange(L)
    rows = od.decode_bf16(inp.pool[inp.block_table[b, j % P], j // P])
    return rows[:, :d_c], rows[:, d_c:]


def _mut_gather_paged_sequence_order(inp, b):
    if inp.wl.layout != "paged":
        return _gather(inp, b)
    P, L, d_c = inp.wl.page_size, int(inp.lens[b]), inp.wl.d_c
    j = np.arange(L)
    rows = od.decode_bf16(inp.pool[inp.block_table.reshape(-1)[j // P], j % P])   # ignores the sequence
    return rows[:, :d_c], rows[:, d_c:]


def _mut_gather_fp8_scale_dropped(inp, b):
    if inp.wl.dtype != "fp8":
        return _gather(inp, b)
    L = int(inp.lens[b])
    return od.decode_e4m3(inp.latent[b, :L]), od.decode_bf16(inp.rope[b, :L])


def _mut_relative_l2_max_norm(x, ref):
    x, ref = np.asarray(x, dtype=np.float64), np.asarray(ref, dtype=np.float64)
    m = ~np.isnan(ref)
    den = np.max(np.abs(ref[m])) if m.any() else 0.0
    num = np.max(np.abs((x - ref)[m])) if m.any() else 0.0
    return float(num / den) if den else float(num)


def _mut_relative_l2_squared(x, ref):
    x, ref = np.asarray(x, dtype=np.float64), np.asarray(ref, dtype=np.float64)
    m = ~np.isnan(ref)
    num, den = np.sum((x - ref)[m] ** 2), np.sum(ref[m] ** 2)
    return float(num / den) if den else float(num)


GATHER_MUTANTS = {
    "packed_columns_swapped": ("gather_rows", _mut_gather_packed_columns_swapped),
    "paged_page_and_slot_swapped": ("gather_rows", _mut_gather_paged_index_transposed),
    "paged_ignores_sequence": ("gather_rows", _mut_gather_paged_sequence_order),
    "fp8_scale_dropped": ("gather_rows", _mut_gather_fp8_scale_dropped),
    "relative_l2_max_norm": ("relative_l2", _mut_relative_l2_max_norm),
    "relative_l2_squared": ("relative_l2", _mut_relative_l2_squared),
}


@pytest.mark.parametrize("name", sorted(GATHER_MUTANTS))
def test_planted_gather_and_metric_mistakes_are_caught(name, monkeypatch):
    attr, fn = GATHER_MUTANTS[name]
    monkeypatch.setattr(od, attr, fn)
    failures = 0
    for chk in (check_gather_rows_hand_placed, check_relative_l2_hand_cases):
        try:
            chk()
        except (AssertionError, ValueError, IndexError):
            failures += 1
    assert failures >= 1, f"planted mistake {name!r} passed every pin"
