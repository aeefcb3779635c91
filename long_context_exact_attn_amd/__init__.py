"""Blockwise exact ring attention for one MI355X (gfx950)."""
