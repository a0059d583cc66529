"""Exact tiled attention for AMD Instinct MI355X (gfx950).

The compute path is libfa.so (hand-written HIP kernels behind a C ABI,
declared in include/fa.h); this package is its Python binding.
"""
from .binding import (FAError, fa_bwd, fa_bwd_dropout, fa_bwd_kvpacked,  # noqa: F401
                      fa_bwd_qkvpacked, fa_bwd_varlen, fa_bwd_varlen_dropout, fa_fwd, fa_fwd_dropout,
                      fa_fwd_fp8, fa_fwd_kvcache, fa_fwd_kvcache_noalloc, fa_fwd_kvpacked, fa_fwd_qkvpacked, fa_fwd_varlen,
                      fa_fwd_varlen_dropout, lib, profiler_disable, profiler_enable, profiler_read,
                      profiler_reset)

__all__ = ["fa_fwd", "fa_bwd", "fa_fwd_varlen", "fa_bwd_varlen", "fa_fwd_kvcache",
           "fa_fwd_dropout", "fa_bwd_dropout", "fa_fwd_varlen_dropout", "fa_bwd_varlen_dropout",
           "fa_fwd_qkvpacked", "fa_bwd_qkvpacked", "fa_fwd_kvpacked", "fa_bwd_kvpacked", "fa_fwd_fp8",
           "fa_fwd_kvcache_noalloc",
           "lib", "FAError", "profiler_enable", "profiler_disable", "profiler_reset", "profiler_read"]
