"""Sparse decode attention with a tail estimate, native to MI355X (gfx950)."""
