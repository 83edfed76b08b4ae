"""CPU oracle of the decoder-only forward (test infrastructure only)."""
