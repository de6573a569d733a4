"""CPU fp64 oracle (test infrastructure only; see hattn_oracle.py)."""
