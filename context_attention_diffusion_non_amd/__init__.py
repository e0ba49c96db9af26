"""cpattn: per-rank context-parallel attention for AMD MI355X (gfx950)."""
