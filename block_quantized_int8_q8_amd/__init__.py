"""Block-quantized int8 MMQ for MI355X (gfx950)."""
