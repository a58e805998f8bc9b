"""CPU oracle (test infrastructure only; see svdq_oracle's header)."""
