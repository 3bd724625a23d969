"""Hybrid Linear Temporal Attention (SWA + DSWA + gated-delta GLA) for MI355X.

The compute lives in ``libhta.so`` (hand-written HIP for gfx950, C ABI declared
in ``include/hta.h``). Submodules:
  ``hta``     the thin ctypes binding, entry points named as in the C ABI;
  ``inputs``  seeded synthetic workloads (shapes and value distributions);
  ``build``   compiles libhta.so in-tree with hipcc.
"""
