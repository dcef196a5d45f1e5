"""Seeded synthetic inputs shared by the oracle-side tests and the GPU harness."""
