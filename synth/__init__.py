"""Seeded synthetic workloads shared by the oracle, the tests and the benchmark."""
