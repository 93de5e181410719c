"""CPU oracle package (test infrastructure only; see moe_oracle)."""
