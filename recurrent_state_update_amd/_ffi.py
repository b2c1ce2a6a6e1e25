"""ctypes declarations of the C ABI in include/mamba2_pool.h."""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, c_char_p, c_int32, c_int64, c_uint64, c_void_p

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmamba2pool.so")

M2_F32, M2_BF16 = 0, 1
STATUS = {0: "M2_OK", 1: "M2_ERR_ARG", 2: "M2_ERR_SHAPE", 3: "M2_ERR_DTYPE", 4: "M2_ERR_ALIGN",
          5: "M2_ERR_SLOT", 6: "M2_ERR_UNSUPPORTED", 7: "M2_ERR_HIP", 8: "M2_ERR_WORKSPACE"}


class PoolDesc(ctypes.Structure):
    _fields_ = [("num_layers", c_int32), ("num_slots", c_int32), ("nheads", c_int32),
                ("head_dim", c_int32), ("d_state", c_int32), ("n_groups", c_int32),
                ("conv_kernel", c_int32), ("ssm_dtype", c_int32), ("conv_dtype", c_int32),
                ("family", c_int32), ("ssm_base", c_void_p), ("conv_base", c_void_p),
                ("ssm_bytes", c_uint64), ("conv_bytes", c_uint64)]


class LayerParams(ctypes.Structure):
    _fields_ = [("A", c_void_p), ("D", c_void_p), ("dt_bias", c_void_p), ("conv_w", c_void_p),
                ("conv_b", c_void_p)]


class Int8StoreDesc(ctypes.Structure):
    _fields_ = [("num_entries", c_int32), ("reserved", c_int32), ("codes", c_void_p), ("scales", c_void_p),
                ("conv", c_void_p), ("codes_bytes", c_uint64), ("scales_bytes", c_uint64),
                ("conv_bytes", c_uint64)]


class Mamba2Error(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status
        self.status_name = STATUS.get(status, str(status))


_IP = POINTER(c_int32)
_SIGS = {
    "mamba2_abi_version": (c_int32, []),
    "mamba2_last_error": (c_char_p, []),
    "mamba2_pool_create": (c_int32, [POINTER(PoolDesc), POINTER(c_void_p)]),
    "mamba2_pool_destroy": (None, [c_void_p]),
    "mamba2_pool_info": (c_int32, [c_void_p, POINTER(c_uint64), POINTER(c_uint64)]),
    "mamba2_decode_step": (c_int32, [c_void_p, c_int32, POINTER(LayerParams), c_int32, c_void_p, c_void_p,
                                     c_void_p, c_int64, c_void_p, c_int64, c_void_p, c_int64, c_void_p, c_int64,
                                     c_void_p, c_int64, c_int32, c_void_p, c_int64, c_int32, c_void_p]),
    "mamba2_prefill_workspace_size": (c_int32, [c_void_p, c_int32, c_void_p, c_void_p, c_int32, c_int32, c_void_p,
                                                c_int32, POINTER(c_uint64)]),
    "mamba2_prefill_chunked": (c_int32, [c_void_p, c_int32, POINTER(LayerParams), c_int32, c_void_p, c_void_p,
                                         c_void_p, c_void_p, c_void_p, c_int64, c_void_p, c_int64, c_void_p,
                                         c_int64, c_void_p, c_int64, c_void_p, c_int64, c_int32, c_void_p,
                                         c_int64, c_int32, c_int32, c_int32, c_void_p, c_int32, c_void_p,
                                         c_uint64, c_void_p]),
    "mamba2_prefill_chunked_noalloc": (c_int32, [c_void_p, c_int32, POINTER(LayerParams), c_int32, c_void_p,
                                                 c_void_p, c_void_p, c_void_p, c_void_p, c_int64, c_void_p, c_int64,
                                                 c_void_p, c_int64, c_void_p, c_int64, c_void_p, c_int64, c_int32,
                                                 c_void_p, c_int64, c_int32, c_int32, c_int32, c_void_p, c_int32,
                                                 c_void_p]),
    "mamba2_checkpoint_states": (c_int32, [c_void_p, c_int32, c_int32, c_void_p, c_void_p, c_void_p, c_void_p,
                                           c_void_p]),
    "mamba2_decode_multi": (c_int32, [c_void_p, c_int32, POINTER(LayerParams), c_int32, c_int32, c_void_p,
                                      c_void_p, c_void_p, c_void_p, c_void_p, c_int64, c_void_p, c_int64, c_void_p,
                                      c_int64, c_void_p, c_int64, c_void_p, c_int64, c_int32, c_void_p, c_int64,
                                      c_int32, c_void_p]),
    "mamba1_decode_step": (c_int32, [c_void_p, c_int32, POINTER(LayerParams), c_int32, c_void_p, c_void_p,
                                     c_void_p, c_int64, c_void_p, c_int64, c_void_p, c_int64, c_void_p, c_int64,
                                     c_void_p, c_int64, c_int32, c_void_p, c_int64, c_int32, c_void_p]),
    "mamba1_prefill_workspace_size": (c_int32, [c_void_p, c_int32, c_int32, c_int32, c_int32,
                                                POINTER(c_uint64)]),
    "mamba1_prefill": (c_int32, [c_void_p, c_int32, POINTER(LayerParams), c_int32, c_void_p, c_void_p,
                                 c_void_p, c_void_p, c_void_p, c_int64, c_void_p, c_int64, c_void_p,
                                 c_int64, c_void_p, c_int64, c_void_p, c_int64, c_int32, c_void_p,
                                 c_int64, c_int32, c_int32, c_int32, c_void_p, c_int32, c_void_p,
                                 c_uint64, c_void_p]),
    "mamba2_int8_store_size": (c_int32, [c_void_p, c_int32, POINTER(c_uint64), POINTER(c_uint64),
                                         POINTER(c_uint64)]),
    "mamba2_int8_store_put": (c_int32, [c_void_p, POINTER(Int8StoreDesc), c_int32, c_int32, c_void_p, c_void_p,
                                        c_void_p, c_void_p, c_void_p]),
    "mamba2_int8_store_get": (c_int32, [c_void_p, POINTER(Int8StoreDesc), c_int32, c_int32, c_void_p, c_void_p,
                                        c_void_p, c_void_p, c_void_p]),
}

_lib = None


def lib() -> ctypes.CDLL:
    """Load libmamba2pool.so (built in-tree); raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built: run `python -m recurrent_state_update_amd.build`")
        l = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(l, name)
            f.restype = res
            f.argtypes = args
        _lib = l
    return _lib


def check(status: int) -> None:
    if status != 0:
        msg = lib().mamba2_last_error()
        raise Mamba2Error(status, msg.decode() if msg else "")


def exported_symbols():
    return list(_SIGS)
