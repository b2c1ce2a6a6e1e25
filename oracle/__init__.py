"""CPU oracle (test infrastructure only; see oracle/mamba2.py)."""
from .mamba2 import (PoolRef, conv_tokens, decode_step, prefill, round_to, silu, softplus, ssd_matrix_form,
                     ssm_scan)

__all__ = ["PoolRef", "conv_tokens", "decode_step", "prefill", "round_to", "silu", "softplus", "ssd_matrix_form",
           "ssm_scan"]
