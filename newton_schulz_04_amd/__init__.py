"""Batched Newton-Schulz orthogonalization for MI355X (gfx950).

The work runs in the HIP library libns.so (C ABI, include/ns.h); this package
only marshals arguments to it. Importing the package does not load the
library; the first call does, and fails loudly if it has not been built.
"""
