"""Compressed Sparse / Heavily Compressed Attention hot path for AMD MI355X (gfx950).

The compute lives in libcsa.so (HIP kernels behind the C ABI of include/csa.h);
`compressed_attention_long_amd.ops` is the thin Python binding over it.
"""
from . import _lib as ops  # noqa: F401
from ._lib import Cache, CsaError  # noqa: F401

__all__ = ["ops", "Cache", "CsaError"]
