"""On-the-fly block-sparse self-attention for video DiTs on MI355X (gfx950)."""
