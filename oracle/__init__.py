"""CPU fp64 reference checker for the MoM layer (test infrastructure only)."""
