"""Hybrid Linear Temporal Attention (SWA + DSWA + gated-delta GLA) for MI355X.

The compute lives in ``libhta.so`` (hand-written HIP for gfx950, C ABI declared
in ``include/hta.h``). ``hybrid_linear_temporal_hta_amd.hta`` is the thin ctypes
binding with the same entry-point names; it is imported lazily so that the
input generator can be used on machines without the built library.
"""
__all__ = ["inputs", "hta"]


def __getattr__(name):
    if name == "hta":
        from . import hta as _hta
        return _hta
    if name == "inputs":
        from . import inputs as _inputs
        return _inputs
    raise AttributeError(name)
