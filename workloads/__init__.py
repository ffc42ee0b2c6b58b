"""Seeded synthetic inputs shared by the tests, the benchmark and the oracle checks."""
