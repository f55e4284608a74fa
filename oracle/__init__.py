"""CPU oracle of the KPool-indexed DSA forward (test infrastructure only; never
imported by the product path)."""
