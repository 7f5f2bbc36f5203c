"""Exact IO-aware attention for MI355X (gfx950): tiled causal prefill and split-KV
paged decode behind a C-ABI library (``libattn.so``).

``exact_io_aware_prefill_amd.attn`` is the thin ctypes binding to that library
(same entry-point names as ``include/attn.h``); importing it raises if the
library has not been built.  ``exact_io_aware_prefill_amd.workloads`` holds the
seeded synthetic input generators.
"""
__all__ = ["attn", "workloads"]
