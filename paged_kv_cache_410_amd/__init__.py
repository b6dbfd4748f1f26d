"""Paged KV-cache decode attention for MI355X (gfx950)."""
