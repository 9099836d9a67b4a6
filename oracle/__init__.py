"""CPU oracle of the multipole gravity evaluation -- test infrastructure only."""
