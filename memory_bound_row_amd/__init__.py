"""Fused LayerNorm forward/backward for AMD MI355X (gfx950)."""
