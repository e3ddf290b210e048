"""CPU oracle of the DSpark sampling / verification engine (test infrastructure only)."""
