"""MI355X (gfx950) library for the absorbed decode step of Multi-Head Latent Attention.

The compute lives in libmla_amd.so (HIP kernels behind the C ABI of include/mla.h); ``ops``
binds it to torch device tensors.  Build with ``python -m mla_latent_kv_attn_amd.build``.
"""
from ._lib import (MLA_BF16, MLA_F32, MLA_FP8_E4M3, MlaError, MlaLibraryError, lib)  # noqa: F401

__all__ = ["lib", "MlaError", "MlaLibraryError", "MLA_F32", "MLA_BF16", "MLA_FP8_E4M3"]
