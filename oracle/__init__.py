"""CPU oracle of the LSA token-selection path (test infrastructure; see lsa_ref.c)."""
