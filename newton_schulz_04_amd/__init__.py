"""Batched Newton-Schulz orthogonalization for MI355X (gfx950).

The work runs in the HIP library libns.so (C ABI, include/ns.h); this package
only marshals arguments to it. Importing the package does not load the
library; the first call does, and raises if it has not been built.
"""
from ._binding import (NOALLOC_SCRATCH_BYTES, NS_BF16, NS_FP32, QUINTIC, NSError, compute_cost,  # noqa: F401
                       last_error, lib, orthogonalize, orthogonalize_chunked,
                       orthogonalize_chunked_raw, orthogonalize_raw, plan_classify, plan_ranks,
                       plan_tiles, profile_enable, profile_read, release_workspace,
                       version, workspace_bytes)
