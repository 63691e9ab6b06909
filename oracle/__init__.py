"""CPU oracle of the HSA decode step (test infrastructure only; see hsa_oracle)."""
