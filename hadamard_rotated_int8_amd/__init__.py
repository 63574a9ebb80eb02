"""Hadamard-rotated INT8 quantized linear layer for AMD Instinct MI355X (gfx950)."""
