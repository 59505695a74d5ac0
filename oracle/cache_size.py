"""Cache-size formulas of the four attention families (test infrastructure only).

Values cached per token per layer, as tabulated on "Grouped-query and latent
attention" (section "Comparison") and "DeepSeek MLA: 4 Attention Methods
Compared" (sections "MHA: one K and V pair for every head", "MQA: share one
K/V head", "GQA: the compromise between MHA and MQA", "Decoupled RoPE"):

  MHA  2 * heads * head_dim
  GQA  2 * groups * head_dim
  MQA  2 * head_dim
  MLA  d_c + d_R         (one joint latent plus the shared rope key)

"MLA storage: Representing KV with a small latent vector", section "Cache
growth with token count", gives the stored total for one request and layer as
T * (d_c + d_R).  Memory is values * layers * tokens * batch * bytes per value.
"""
from __future__ import annotations


def mha_values(heads: int, head_dim: int) -> int:
    return 2 * heads * head_dim


def gqa_values(groups: int, head_dim: int) -> int:
    return 2 * groups * head_dim


def mqa_values(head_dim: int) -> int:
    return 2 * head_dim


def mla_values(d_c: int, d_R: int) -> int:
    return d_c + d_R


def stored_components(tokens: int, values_per_token: int) -> int:
    """Components held for one request in one layer after ``tokens`` tokens."""
    return tokens * values_per_token


def cache_bytes(values_per_token: int, layers: int, tokens: int, batch: int = 1,
                bytes_per_value: int = 2) -> int:
    return values_per_token * layers * tokens * batch * bytes_per_value


def cache_gib(values_per_token: int, layers: int, tokens: int, batch: int = 1,
              bytes_per_value: int = 2) -> float:
    return cache_bytes(values_per_token, layers, tokens, batch, bytes_per_value) / float(1024 ** 3)
