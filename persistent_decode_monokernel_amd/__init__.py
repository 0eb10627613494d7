"""Batch-1 persistent decode monokernel for MI355X (gfx950).

The product is ``libkie.so`` (C ABI in ``include/kie.h``): HIP kernels that
run every decode step of an fp16 decoder-only transformer inside one
persistent launch.  This package is its thin Python binding.
"""
from ._lib import KieError, STATUS, declared_functions, load
from .engine import Engine, config_check, debug_barrier, debug_gemm, debug_gemv, debug_stream, make_config

__all__ = ["Engine", "KieError", "STATUS", "config_check", "debug_barrier", "debug_gemm", "debug_gemv",
           "debug_stream", "declared_functions", "load", "make_config"]
