"""Routed mixture-of-experts with block-scaled 4-bit expert weights on MI355X (gfx950)."""
