"""The five synthetic decode workloads (shapes, dtypes, layouts, seeds).

Dimensions follow the DeepSeek-V3 numbers quoted on "Grouped-query and latent
attention" (section "Multi-head latent attention (MLA)": 128 heads, 128-wide
content keys and values, a 512-wide latent) and "DeepSeek MLA: 4 Attention
Methods Compared" (section "DeepSeek MLA dimensions from the official
implementation": kv_lora_rank 512, qk_rope_head_dim 64, v_head_dim 128).
The batch sizes, lengths, page size and fp8 format are synthetic serving
workloads chosen for this library, not values from the pages.
"""
from __future__ import annotations

from dataclasses import dataclass, field


@dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    B: int                 # sequences in the batch
    H: int                 # query heads
    d_h: int               # content key / value width per head (d_v == d_h)
    d_c: int               # latent width
    d_R: int               # decoupled rope key width
    n_max: int             # cache capacity per sequence (tokens)
    len_lo: int            # sequence lengths are uniform integers in [len_lo, len_hi]
    len_hi: int
    dtype: str             # "f32" | "bf16" | "fp8"  (storage type of the latent cache)
    layout: str            # "split" | "packed" | "paged"
    page_size: int = 64
    rope_base: float = 10000.0
    description: str = field(default="", compare=False)

    @property
    def w_std(self) -> float:
        # weights ~ N(0, 1/d_c): variance 1/d_c
        return (1.0 / self.d_c) ** 0.5

    @property
    def scale(self) -> float:
        return 1.0 / float(self.d_h + self.d_R) ** 0.5

    def with_(self, **kw) -> "Workload":
        d = self.__dict__.copy()
        d.update(kw)
        return Workload(**d)


WORKLOADS = {
    1: Workload("tiny-f32", seed=1, B=1, H=4, d_h=16, d_c=32, d_R=8, n_max=64,
                len_lo=64, len_hi=64, dtype="f32", layout="split",
                description="tiny fp32 decode, B=1 H=4 d_h=16 d_c=32 d_R=8 N=64"),
    2: Workload("v3-b1", seed=2, B=1, H=128, d_h=128, d_c=512, d_R=64, n_max=4096,
                len_lo=4096, len_hi=4096, dtype="bf16", layout="split",
                description="V3-shape decode, B=1 N=4096 bf16 split latent/rope caches"),
    3: Workload("v3-b64-var", seed=3, B=64, H=128, d_h=128, d_c=512, d_R=64, n_max=8192,
                len_lo=1024, len_hi=8192, dtype="bf16", layout="packed",
                description="V3-shape decode, B=64 lengths U[1024,8192], packed [B,8192,576] bf16"),
    4: Workload("v3-paged-32k", seed=4, B=16, H=128, d_h=128, d_c=512, d_R=64, n_max=32768,
                len_lo=32768, len_hi=32768, dtype="bf16", layout="paged", page_size=64,
                description="V3-shape decode, B=16 N=32768, 64-token pages, permuted block table"),
    5: Workload("v3-fp8", seed=5, B=128, H=128, d_h=128, d_c=512, d_R=64, n_max=16384,
                len_lo=2048, len_hi=16384, dtype="fp8", layout="split",
                description="V3-shape decode, B=128 lengths U[2048,16384], e4m3 latents + fp32 scale"),
}


def get_workload(key) -> Workload:
    if isinstance(key, Workload):
        return key
    if isinstance(key, int):
        return WORKLOADS[key]
    for w in WORKLOADS.values():
        if w.name == key:
            return w
    raise KeyError(key)
