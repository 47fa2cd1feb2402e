"""Sparse mixture-of-experts FFN layer for AMD Instinct MI355X (gfx950).

The layer runs in hand-written HIP kernels behind the C ABI declared in
``include/moe_layer.h`` (``libmoe_layer.so``); this package holds the kernels'
sources (``csrc/``), the build script and a ctypes binding.
"""
from .moe import (FLAG_FORCE_GEMM, FLAG_FORCE_GEMV, MoeError, forward, lib, route,  # noqa: F401
                  workspace_size)
