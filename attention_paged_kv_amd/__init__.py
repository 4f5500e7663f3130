"""Paged-KV causal attention for AMD MI355X (gfx950)."""
