"""fp64 CPU oracle of the QEvict decode hot path (test infrastructure only)."""
