"""Causal packed flash attention for MI355X (gfx950): Python binding of the C-ABI library."""
