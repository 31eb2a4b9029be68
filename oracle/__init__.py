"""CPU oracle -- test infrastructure only (see moe_oracle)."""
