"""Seeded synthetic inputs (random draws and layout only, no method arithmetic)."""
