"""libfa: exact, tiled, fused attention for MI355X (gfx950)."""
