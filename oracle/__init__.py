"""CPU oracle for the GQE forward pass -- test infrastructure only (see gqe_oracle.py)."""
