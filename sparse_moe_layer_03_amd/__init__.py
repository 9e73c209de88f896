"""Sparse Mixture-of-Experts FFN layer for one AMD Instinct MI355X (gfx950)."""
