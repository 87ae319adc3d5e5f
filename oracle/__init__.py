"""fp64 CPU oracle of the IP-TTCD layer forward (test infrastructure only)."""
