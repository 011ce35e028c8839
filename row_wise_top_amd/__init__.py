"""Row-wise top-k selection on MI355X (gfx950)."""
