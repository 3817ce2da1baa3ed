"""Float64 CPU oracle (test infrastructure only; never used by the GPU path)."""
