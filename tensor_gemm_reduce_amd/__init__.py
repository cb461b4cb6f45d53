"""Fused BF16 GEMM + reduce-scatter for AMD Instinct MI355X (gfx950).

One rank's share of a tensor-parallel row-parallel linear layer, computed by a
single persistent HIP kernel: compute workgroups run the MFMA GEMM and route
finished tiles into per-destination slice buffers with ready flags; reducer
workgroups sum this rank's slice with the peer partials as tiles are flagged.

The C ABI is ``include/gemm_rs.h`` (``libgemm_rs.so``); ``gemm_rs`` is its
ctypes binding.
"""
from .gemm_rs import (  # noqa: F401
    GemmRS, GemmRSError, gemm_rs_config, gemm_rs_info, make_config,
    gemm_rs_validate, gemm_rs_plan, gemm_rs_plan_slots, gemm_rs_create, gemm_rs_run,
    gemm_rs_status, gemm_rs_query, gemm_rs_debug_read, gemm_rs_destroy, gemm_rs_strerror,
    MODE_FUSED, MODE_GEMM_ONLY, MODE_REDUCE_ONLY, MODE_SEQUENTIAL,
)
