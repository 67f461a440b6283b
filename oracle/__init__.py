"""CPU oracle of the MatMul-free LM block forward (test infrastructure only)."""
