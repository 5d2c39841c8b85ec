"""fp64 CPU oracle (test infrastructure only; see oracle.py and gla_oracle.c)."""
