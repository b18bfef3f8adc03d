"""Seeded synthetic input generators shared by the tests and the benchmark."""
