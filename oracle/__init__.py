"""CPU oracle of the TurboQuant codec -- test infrastructure only (see tq_oracle)."""
