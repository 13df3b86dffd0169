"""Seeded synthetic inputs and workload shapes (no attention arithmetic)."""
