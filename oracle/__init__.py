"""CPU oracle (test infrastructure only; see masw_oracle.py's header)."""
