"""CPU oracle (test infrastructure only): see oracle/moe_oracle.py."""
