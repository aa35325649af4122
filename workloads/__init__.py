"""Seeded synthetic input generators (no method arithmetic)."""
