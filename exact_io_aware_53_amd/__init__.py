"""Exact IO-aware attention for MI355X (gfx950): Python binding of libfa.so."""
