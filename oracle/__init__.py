"""CPU oracle (test infrastructure only; see turbokv_oracle)."""
