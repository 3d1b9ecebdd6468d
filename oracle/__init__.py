"""fp64 CPU oracle of the selective scan -- test infrastructure only (see oracle.py)."""
