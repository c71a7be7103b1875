"""CPU oracle (test infrastructure only): see anchorkv_oracle.py."""
