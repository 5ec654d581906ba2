"""CPU oracle of the HHR decode path (test infrastructure only; see hhr_oracle)."""
