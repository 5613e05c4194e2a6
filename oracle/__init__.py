"""CPU oracle for the EPLB hot path (test infrastructure only; see eplb_oracle)."""
