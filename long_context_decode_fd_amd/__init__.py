"""Flash-Decoding (split-KV single-query decode attention) for MI355X.

The computation lives in libfd.so (HIP kernels for gfx950 behind the C ABI
declared in include/fd.h); this package is its Python binding plus the
seeded synthetic workloads used by the tests and the benchmark.

    from long_context_decode_fd_amd import fd_decode
    out, lse = fd_decode(q, k_cache, v_cache, seqlens, scale)
"""
from ._binding import (FD_BF16, FD_ERR_CAPTURE, FD_ERR_HIP,  # noqa: F401
                       FD_ERR_INVALID_ARG, FD_ERR_TOO_LARGE,
                       FD_ERR_UNSUPPORTED, FD_ERR_WORKSPACE, FD_F16, FD_F32,
                       FD_FLAG_FUSED_MERGE, FD_FLAG_PARTIALS,
                       FD_FLAG_UNIFIED_MAX, FD_MERGE_FUSED,
                       FD_MERGE_NONE,
                       FD_MERGE_SEPARATE, FD_OK, FD_PAGES_HEAD_MAJOR,
                       FD_PAGES_TOKEN_MAJOR, FD_PARTIALS_CHUNK_MAJOR,
                       FD_PARTIALS_ROW_MAJOR,
                       FD_VARIANT_AUTO, FD_VARIANT_MFMA, FD_VARIANT_VALU,
                       LIB_PATH, NOALLOC_SCRATCH_BYTES, FdError, fd_decode,
                       fd_decode_ex, fd_decode_noalloc,
                       fd_decode_multiquery, fd_decode_paged,
                       fd_decode_unified_max,
                       fd_decode_partials, fd_merge_partials, fd_plan,
                       fd_plan_ex, fd_status_string, fd_version,
                       fd_workspace_bytes, load_library)
