"""CPU oracle for the Quest decode step (test infrastructure only)."""
