"""Seeded synthetic inputs (shared by the oracle side and the GPU side)."""
