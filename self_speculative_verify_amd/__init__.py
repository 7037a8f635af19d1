"""Fused quantized weight sweep for MI355X (gfx950).

The sweep runs in ``libqgemm.so`` (hand-written HIP kernels behind a C ABI,
``include/qgemm.h``); ``qgemm`` is its Python binding.
"""
from . import qgemm  # noqa: F401
