"""Mamba2 selective-state update over a slot pool: binding of the MI355X (gfx950) HIP library.

Importing the package loads nothing; the shared library is loaded on first
use of Pool (recurrent_state_update_amd.pool) and raises if it is not built.
"""

__all__ = ["Pool", "LayerWeights", "Mamba2Error"]


def __getattr__(name):
    if name in __all__:
        from . import pool
        return getattr(pool, name)
    raise AttributeError(name)
