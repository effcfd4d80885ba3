"""libattn: fused attention forward and block-sparse backward for MI355X (gfx950)."""
