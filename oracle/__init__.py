"""CPU oracle (test infrastructure only; see kvc_oracle)."""
