"""Position-independent KV-cache reuse on AMD Instinct MI355X (gfx950).

The work happens in libpic.so (hand-written HIP kernels behind a C ABI,
declared in include/pic.h).  This package is a thin ctypes binding: it
marshals arguments and raises on error codes; every step of the hot path runs
in the library's kernels.  PyTorch supplies device memory and streams only.
"""
from .binding import (  # noqa: F401
    PIC_BF16, PIC_F32, TARGET_AUTO, TARGET_ORIGINAL, KEYS_ROTATED, KEYS_UNROTATED, VARIANT_FUSED,
    VARIANT_MATERIALIZED,
    PLAN_ONLY, DRY_RUN, DEFER_GATHER, QUERY_ROTATION, VALUES_IN_POOL, PicError, Plan, Pool, Store, lib, library_path,
    model_struct, write_chunk_file,
)
