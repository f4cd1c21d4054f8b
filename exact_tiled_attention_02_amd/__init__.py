"""Exact tiled attention (FlashAttention-2 forward and backward) for MI355X (gfx950)."""
