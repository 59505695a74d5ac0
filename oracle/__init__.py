"""CPU oracle for MLA absorbed decode -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path (the HIP library and
its Python binding) never imports, links or calls it, and it imports nothing
from the product path: it shares no code, tables or helpers with the kernels.

The oracle computes the plain, non-absorbed definition of one decode step:
rebuild every cached token's per-head key [W_UK c ; k_R] and value W_UV c
explicitly, then run ordinary softmax attention for the single new query with
scale 1/sqrt(d_h + d_R).  Arithmetic is float64 unless a caller asks for
float32.

Parity status of each function (what pins it, see tests/test_oracle_pins.py):
  expand_kv        pinned: worked example of "MLA storage: Representing KV with
                   a small latent vector" (keys [1,2],[2,3]; values [4,2],[1,5]).
  attend / decode  pinned: closed forms (one token, zero query, two tokens),
                   torch scaled_dot_product_attention on explicit K/V, the
                   absorption identities of "Grouped-query and latent attention".
  merge_partials   pinned: equals one-pass softmax for every split of the tokens.
  cache_size.*     pinned: every cache-size figure printed on the pages.
  cache_write.*    pinned: closed forms and invariants of the cache write (the new
                   token's latent W_DKV h and rotated rope key RoPE_pos(W_KR h), and
                   their bf16 / E4M3 storage forms), tests/test_oracle_cache_write.py.
  query.*          pinned: basis vectors and head slices of the query projections, single
                   rotary components per head, the relative-position property against the
                   cache write's k_R, a hand-computed fold, the fold against explicit keys,
                   tests/test_oracle_query.py.
  output.*         pinned: basis vectors of W_O, a hand-computed fold, and the folded product
                   against W_O of the explicit-value decode, tests/test_oracle_output.py.
  decode_bf16 / decode_e4m3  pinned: OCP FP8 special values, bf16 bit patterns.
  The rotary pairing convention of the input generator is not fixed by the
  pages: parity unpinned for that convention (both sides consume the same
  already-rotated bytes, so parity does not depend on it).
"""
from .mla_decode import (  # noqa: F401
    decode_bf16, decode_e4m3, gather_rows, expand_kv, attend, decode,
    merge_partials, relative_l2,
)
from . import cache_size  # noqa: F401
from . import cache_write  # noqa: F401
from . import query  # noqa: F401
from . import output  # noqa: F401
