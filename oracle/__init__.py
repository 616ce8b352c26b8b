"""CPU oracle for the sparse MoE layer forward (test infrastructure only)."""
