"""Load-balanced context-parallel causal attention and GQA decode for MI355X (gfx950)."""
