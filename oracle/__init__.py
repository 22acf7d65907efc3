"""fp64 CPU oracle for Newton-Schulz orthogonalization (test infrastructure)."""
