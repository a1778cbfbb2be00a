"""CPU oracle for the Engram forward hot path (test infrastructure only)."""
