"""Mamba2 selective-state update over a slot pool, MI355X (gfx950) HIP library binding."""
