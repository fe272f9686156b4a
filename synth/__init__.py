"""Seeded synthetic input generators (random draws only, no method arithmetic)."""
