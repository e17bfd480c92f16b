"""CPU oracle of the ANVIL bank step: test infrastructure only (see anvil_oracle.py)."""
