"""Paged Q8_0/Q4_0 attention for MI355X (gfx950): Python binding of libkvattn.so."""
