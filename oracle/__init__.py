"""fp64 CPU oracle for fused linear cross-entropy: test infrastructure only."""
