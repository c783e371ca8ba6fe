"""CPU oracle of the CSA layer: test infrastructure only (see csa_oracle's header)."""
