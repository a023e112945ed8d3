"""W4A16 weight-only-quantized linear layer for MI355X (gfx950)."""
