"""fp64 CPU oracle for the log-linear token mixer (test infrastructure only)."""
