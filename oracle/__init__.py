"""fp64 CPU oracle of the fused chunked KL loss (test infrastructure only)."""
