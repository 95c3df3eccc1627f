"""Multi-scale retention (parallel, recurrent and chunkwise forms, per-head GroupNorm) for MI355X.

The computation runs in hand-written gfx950 HIP kernels inside libretention.so, reached through
the C ABI declared in include/retention.h. This package is the thin ctypes binding over it
(`retention`), the seeded input generators (`inputs`), and the build step (`build`).
"""
from .retention import (GroupNorm, RetentionError, chunkwise_fwd, load_library, parallel_fwd,  # noqa: F401
                        recurrent_step, workspace_bytes)

__all__ = ["GroupNorm", "RetentionError", "chunkwise_fwd", "load_library", "parallel_fwd", "recurrent_step",
           "workspace_bytes"]
