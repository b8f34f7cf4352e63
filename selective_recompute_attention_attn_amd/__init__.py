"""Selective-recompute attention core and sequence-parallel norm region for MI355X.

The compute lives in ``libsrat.so`` (hand-written HIP for gfx950 behind a C
ABI declared in ``include/srat.h``); this package only marshals arguments.
Importing it loads nothing: the library is opened on first use.
"""
import importlib

__all__ = ["attn_core_fwd", "attn_core_bwd", "sp_norm_fwd", "sp_norm_bwd"]


def __getattr__(name):
    if name in __all__:
        return getattr(importlib.import_module(__name__ + ".ops"), name)
    raise AttributeError(name)
