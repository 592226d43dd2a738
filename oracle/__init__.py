"""CPU fp64 oracle -- test infrastructure only (see oracle.py)."""
