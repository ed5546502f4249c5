"""CPU oracle for the Engram layer: test infrastructure only (see engram_oracle)."""
