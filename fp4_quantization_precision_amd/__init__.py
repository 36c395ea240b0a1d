"""libtq: block-scaled FP4 (NVFP4-style) quantisation for MI355X (gfx950)."""
