"""fp64 CPU oracle for the MapFlow hot path (test infrastructure only)."""
