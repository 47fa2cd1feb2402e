"""Seeded synthetic inputs shared by the oracle and the GPU path (no layer arithmetic)."""
