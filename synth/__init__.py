"""Seeded synthetic inputs shared by the HIP path tests and the oracle (no method arithmetic)."""
