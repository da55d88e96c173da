"""CPU oracle of the DSpine draft-block hot path (test infrastructure only)."""
