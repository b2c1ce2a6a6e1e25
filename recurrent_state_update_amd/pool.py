"""Torch-facing binding of libmamba2pool.so: argument marshalling only.

Tensors supply device pointers, dtypes and row strides; the stream is
torch's current stream.  Every computation runs in the HIP kernels of the
library, and a missing library raises instead of falling back to anything.
"""
from __future__ import annotations

import ctypes
from ctypes import byref, c_uint64, c_void_p

import numpy as np
import torch

from ._ffi import M2_BF16, M2_F32, Int8StoreDesc, LayerParams, Mamba2Error, PoolDesc, check, lib

_DT = {torch.float32: M2_F32, torch.bfloat16: M2_BF16}


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype not in _DT:
        raise TypeError(f"unsupported dtype {t.dtype}; use float32 or bfloat16")
    return _DT[t.dtype]


def _rows(t: torch.Tensor, name: str):
    if t.dim() != 2 or t.stride(1) != 1:
        raise ValueError(f"{name} must be a 2-D tensor with a contiguous last dimension")
    return c_void_p(t.data_ptr()), t.stride(0)


def _stream():
    return c_void_p(torch.cuda.current_stream().cuda_stream)


def _host_i32(a):
    if a is None:
        return None, None
    arr = np.ascontiguousarray(np.asarray(a, dtype=np.int32))
    return arr, arr.ctypes.data_as(c_void_p)


class LayerWeights:
    """fp32 device parameters of one layer: A, D, dt_bias [H], conv_w [Cd, W], conv_b [Cd]."""

    def __init__(self, A, D, dt_bias, conv_w, conv_b):
        self.tensors = [t.contiguous() for t in (A, D, dt_bias, conv_w, conv_b)]
        for t in self.tensors:
            if t.dtype != torch.float32:
                raise TypeError("layer parameters must be float32")
        self.A, self.D, self.dt_bias, self.conv_w, self.conv_b = self.tensors
        self.struct = LayerParams(*(t.data_ptr() for t in self.tensors))

    @classmethod
    def from_numpy(cls, p: dict, device="cuda"):
        f = lambda k: torch.as_tensor(np.asarray(p[k], np.float32), device=device)
        return cls(f("A"), f("D"), f("dt_bias"), f("conv_w"), f("conv_b"))


class Pool:
    """Slot pool over caller-owned tensors ssm [L, S, H, P, N] and conv [L, S, Cd, W-1]."""

    def __init__(self, ssm: torch.Tensor, conv: torch.Tensor, nheads: int, head_dim: int, d_state: int,
                 n_groups: int, conv_kernel: int, family: int = 0):
        if not (ssm.is_contiguous() and conv.is_contiguous()):
            raise ValueError("pool tensors must be contiguous")
        self.ssm, self.conv = ssm, conv
        self.nheads, self.head_dim, self.d_state = nheads, head_dim, d_state
        self.n_groups, self.conv_kernel = n_groups, conv_kernel
        self.family = family               # 0: Mamba2, 1: Mamba1 (nheads = D channels, head_dim 1), 2: GDN, 3: KDA
        self.intermediate = nheads * head_dim
        self.conv_dim = self.intermediate + (0 if family == 1 else 2 * n_groups * d_state)
        self.num_layers, self.num_slots = ssm.shape[0], ssm.shape[1]
        desc = PoolDesc(self.num_layers, self.num_slots, nheads, head_dim, d_state, n_groups, conv_kernel,
                        _dtype_code(ssm), _dtype_code(conv), family, ssm.data_ptr(), conv.data_ptr(),
                        ssm.numel() * ssm.element_size(), conv.numel() * conv.element_size())
        h = c_void_p()
        check(lib().mamba2_pool_create(byref(desc), byref(h)))
        self._h = h

    @classmethod
    def allocate(cls, num_layers, num_slots, nheads, head_dim, d_state, n_groups, conv_kernel,
                 ssm_dtype=torch.bfloat16, conv_dtype=torch.bfloat16, device="cuda"):
        cd = nheads * head_dim + 2 * n_groups * d_state
        ssm = torch.zeros((num_layers, num_slots, nheads, head_dim, d_state), dtype=ssm_dtype, device=device)
        conv = torch.zeros((num_layers, num_slots, cd, conv_kernel - 1), dtype=conv_dtype, device=device)
        return cls(ssm, conv, nheads, head_dim, d_state, n_groups, conv_kernel)

    @classmethod
    def allocate_mamba1(cls, num_layers, num_slots, d_inner, d_state, conv_kernel, ssm_dtype=torch.bfloat16,
                        conv_dtype=torch.bfloat16, device="cuda"):
        """A Mamba1 pool: ssm [L, S, D, 1, N] (the (D, N) state) and conv [L, S, D, W-1]."""
        ssm = torch.zeros((num_layers, num_slots, d_inner, 1, d_state), dtype=ssm_dtype, device=device)
        conv = torch.zeros((num_layers, num_slots, d_inner, conv_kernel - 1), dtype=conv_dtype, device=device)
        return cls(ssm, conv, d_inner, 1, d_state, 1, conv_kernel, family=1)

    @classmethod
    def allocate_gdn(cls, num_layers, num_slots, num_v_heads, head_v_dim, head_k_dim, num_k_heads, conv_kernel,
                     device="cuda"):
        """A GDN pool (state only: the pages give no recurrence): ssm [L, S, Hv, dv, dk] and conv
        [L, S, Hv*dv + 2*Hk*dk, W-1], both bf16."""
        cd = num_v_heads * head_v_dim + 2 * num_k_heads * head_k_dim
        ssm = torch.zeros((num_layers, num_slots, num_v_heads, head_v_dim, head_k_dim), dtype=torch.bfloat16,
                          device=device)
        conv = torch.zeros((num_layers, num_slots, cd, conv_kernel - 1), dtype=torch.bfloat16, device=device)
        return cls(ssm, conv, num_v_heads, head_v_dim, head_k_dim, num_k_heads, conv_kernel, family=2)

    @classmethod
    def allocate_kda(cls, num_layers, num_slots, num_heads, head_dim, conv_kernel, device="cuda"):
        """A KDA pool (state only: the pages give no recurrence): ssm [L, S, H, d, d] fp32 and conv
        [L, S, 3*H*d, W-1] bf16."""
        ssm = torch.zeros((num_layers, num_slots, num_heads, head_dim, head_dim), dtype=torch.float32, device=device)
        conv = torch.zeros((num_layers, num_slots, 3 * num_heads * head_dim, conv_kernel - 1), dtype=torch.bfloat16,
                           device=device)
        return cls(ssm, conv, num_heads, head_dim, head_dim, num_heads, conv_kernel, family=3)

    def mamba1_decode_step(self, layer: int, w: LayerWeights, slots: torch.Tensor, x, B, C, z, dt, y,
                           slots_host=None):
        """One Mamba1 token per row of slots (device int32): x, z, dt rows of D, B and C rows of N;
        w.A is the (D, N) decay matrix."""
        if slots.dtype != torch.int32:
            raise TypeError("slots must be int32")
        _, sh_ptr = _host_i32(slots_host)
        io = _dtype_code(x)
        for t in (B, C, z, dt):
            if _dtype_code(t) != io:
                raise TypeError("x, B, C, z and dt must share one dtype")
        xp, xs = _rows(x, "x")
        bp, bs = _rows(B, "B")
        cp, cs = _rows(C, "C")
        zp, zs = _rows(z, "z")
        dp, ds = _rows(dt, "dt")
        yp, ys = _rows(y, "y")
        check(lib().mamba1_decode_step(self._h, layer, byref(w.struct), slots.numel(), c_void_p(slots.data_ptr()),
                                       sh_ptr, xp, xs, bp, bs, cp, cs, zp, zs, dp, ds, io, yp, ys,
                                       _dtype_code(y), _stream()))
        return y

    def mamba1_workspace_size(self, num_seqs: int, total_tokens: int, chunk_size: int = 0,
                              max_ckpt: int = 0) -> int:
        n = c_uint64()
        check(lib().mamba1_prefill_workspace_size(self._h, num_seqs, total_tokens, chunk_size, max_ckpt,
                                                  byref(n)))
        return n.value

    def mamba1_prefill(self, layer: int, w: LayerWeights, cu_seqlens, slots, has_init, x, B, C, z, dt, y,
                       start_pos=None, chunk_size: int = 0, ckpt_interval: int = 0, ckpt_slots=None,
                       workspace: torch.Tensor | None = None):
        """Mamba1 prefill of packed sequences (rows x, z, dt of D; B, C of N); cu_seqlens, slots,
        has_init, start_pos and ckpt_slots [num_seqs][max_ckpt] are host arrays; chunk_size 0 lets
        the library choose the chunking."""
        cu, _ = _host_i32(cu_seqlens)
        sl, sl_p = _host_i32(slots)
        hi = np.ascontiguousarray(np.asarray(has_init, dtype=np.uint8))
        sp, sp_p = _host_i32(start_pos)   # sp keeps the array alive through the call
        ns = len(sl)
        max_ck, ck_p = 0, None
        if ckpt_slots is not None:
            ck = np.ascontiguousarray(np.asarray(ckpt_slots, dtype=np.int32).reshape(ns, -1))
            max_ck = ck.shape[1]
            ck_p = ck.ctypes.data_as(c_void_p)
        total = int(cu[-1]) if len(cu) else 0
        if workspace is None:
            workspace = torch.empty(self.mamba1_workspace_size(ns, total, chunk_size, max_ck), dtype=torch.uint8,
                                    device=self.ssm.device)
        io = _dtype_code(x)
        for t in (B, C, z, dt):
            if _dtype_code(t) != io:
                raise TypeError("x, B, C, z and dt must share one dtype")
        xp, xs = _rows(x, "x")
        bp, bs = _rows(B, "B")
        cp, cs = _rows(C, "C")
        zp, zs = _rows(z, "z")
        dp, ds = _rows(dt, "dt")
        yp, ys = _rows(y, "y")
        check(lib().mamba1_prefill(
            self._h, layer, byref(w.struct), ns, cu.ctypes.data_as(c_void_p), sl_p,
            hi.ctypes.data_as(c_void_p), sp_p, xp, xs, bp, bs, cp, cs, zp, zs, dp, ds, io, yp, ys,
            _dtype_code(y), chunk_size, ckpt_interval, ck_p, max_ck, c_void_p(workspace.data_ptr()),
            workspace.numel(), _stream()))
        return y

    def close(self):
        if getattr(self, "_h", None):
            lib().mamba2_pool_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def info(self):
        s, c = c_uint64(), c_uint64()
        check(lib().mamba2_pool_info(self._h, byref(s), byref(c)))
        return s.value, c.value

    def split_xbc(self, u: torch.Tensor):
        """Views x, B, C of packed pre-conv rows u [rows, Cd]."""
        I, GN = self.intermediate, self.n_groups * self.d_state
        return u[:, :I], u[:, I:I + GN], u[:, I + GN:]

    # ------------------------------------------------------------------ decode
    def decode_step(self, layer: int, w: LayerWeights, slots: torch.Tensor, x, B, C, z, dt, y,
                    slots_host=None):
        """One token per row of slots (device int32); writes y in place and updates the pool."""
        if slots.dtype != torch.int32:
            raise TypeError("slots must be int32")
        _, sh_ptr = _host_i32(slots_host)
        io = _dtype_code(x)
        for t in (B, C, z, dt):
            if _dtype_code(t) != io:
                raise TypeError("x, B, C, z and dt must share one dtype")
        xp, xs = _rows(x, "x")
        bp, bs = _rows(B, "B")
        cp, cs = _rows(C, "C")
        zp, zs = _rows(z, "z")
        dp, ds = _rows(dt, "dt")
        yp, ys = _rows(y, "y")
        check(lib().mamba2_decode_step(self._h, layer, byref(w.struct), slots.numel(), c_void_p(slots.data_ptr()),
                                       sh_ptr, xp, xs, bp, bs, cp, cs, zp, zs, dp, ds, io, yp, ys,
                                       _dtype_code(y), _stream()))
        return y

    def decode_multi(self, layer: int, w: LayerWeights, slots_in: torch.Tensor, slots_out: torch.Tensor,
                     x, B, C, z, dt, y, slots_in_host=None, slots_out_host=None):
        """num_tokens = slots_out.shape[1] decode tokens per row of slots_in (device int32), rows
        b*num_tokens + t of x, B, C, z, dt and y; the state after token t goes to slots_out[b, t]."""
        if slots_in.dtype != torch.int32 or slots_out.dtype != torch.int32:
            raise TypeError("slots must be int32")
        if slots_out.dim() != 2 or slots_out.shape[0] != slots_in.numel() or not slots_out.is_contiguous():
            raise ValueError("slots_out must be a contiguous [batch, num_tokens] tensor")
        _, si_p = _host_i32(slots_in_host)
        _, so_p = _host_i32(None if slots_out_host is None else np.asarray(slots_out_host).reshape(-1))
        io = _dtype_code(x)
        for t in (B, C, z, dt):
            if _dtype_code(t) != io:
                raise TypeError("x, B, C, z and dt must share one dtype")
        xp, xs = _rows(x, "x")
        bp, bs = _rows(B, "B")
        cp, cs = _rows(C, "C")
        zp, zs = _rows(z, "z")
        dp, ds = _rows(dt, "dt")
        yp, ys = _rows(y, "y")
        check(lib().mamba2_decode_multi(self._h, layer, byref(w.struct), slots_in.numel(), slots_out.shape[1],
                                        c_void_p(slots_in.data_ptr()), c_void_p(slots_out.data_ptr()), si_p, so_p,
                                        xp, xs, bp, bs, cp, cs, zp, zs, dp, ds, io, yp, ys, _dtype_code(y),
                                        _stream()))
        return y

    # ------------------------------------------------------------------ prefill
    def workspace_size(self, cu_seqlens, chunk_size: int = 256, start_pos=None, ckpt_interval: int = 0,
                       ckpt_slots=None) -> int:
        """Workspace bytes of a prefill call with these host arguments (the library counts the chunks)."""
        cu, cu_p = _host_i32(cu_seqlens)
        ns = len(cu) - 1
        _, sp_p = _host_i32(start_pos)
        ck_p, max_ck = None, 0
        if ckpt_slots is not None:
            ck = np.ascontiguousarray(np.asarray(ckpt_slots, dtype=np.int32).reshape(ns, -1))
            ck_p, max_ck = ck.ctypes.data_as(c_void_p), ck.shape[1]
        n = c_uint64()
        check(lib().mamba2_prefill_workspace_size(self._h, ns, cu_p, sp_p, chunk_size, ckpt_interval, ck_p, max_ck,
                                                  byref(n)))
        return n.value

    def prefill(self, layer: int, w: LayerWeights, cu_seqlens, slots, has_init, x, B, C, z, dt, y,
                start_pos=None, chunk_size: int = 256, ckpt_interval: int = 0, ckpt_slots=None,
                workspace: torch.Tensor | None = None):
        """Chunked prefill of packed sequences; cu_seqlens/slots/has_init/start_pos/ckpt_slots are host arrays."""
        cu, cu_p = _host_i32(cu_seqlens)
        sl, sl_p = _host_i32(slots)
        hi = np.ascontiguousarray(np.asarray(has_init, dtype=np.uint8))
        sp, sp_p = _host_i32(start_pos)
        ns = len(sl)
        max_ck = 0
        ck_p = None
        if ckpt_slots is not None:
            ck = np.ascontiguousarray(np.asarray(ckpt_slots, dtype=np.int32).reshape(ns, -1))
            max_ck = ck.shape[1]
            ck_p = ck.ctypes.data_as(c_void_p)
        if workspace is None:
            need = self.workspace_size(cu, chunk_size, sp, ckpt_interval, ckpt_slots)
            workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=self.ssm.device)
        io = _dtype_code(x)
        xp, xs = _rows(x, "x")
        bp, bs = _rows(B, "B")
        cp, cs = _rows(C, "C")
        zp, zs = _rows(z, "z")
        dp, ds = _rows(dt, "dt")
        yp, ys = _rows(y, "y")
        check(lib().mamba2_prefill_chunked(
            self._h, layer, byref(w.struct), ns, cu.ctypes.data_as(c_void_p), sl_p,
            hi.ctypes.data_as(c_void_p), sp_p, xp, xs, bp, bs, cp, cs, zp, zs, dp, ds, io, yp, ys,
            _dtype_code(y), chunk_size, ckpt_interval, ck_p, max_ck, c_void_p(workspace.data_ptr()),
            workspace.numel(), _stream()))
        return y

    def prefill_noalloc(self, layer: int, w: LayerWeights, cu_seqlens, slots, has_init, x, B, C, z, dt, y,
                        start_pos=None, chunk_size: int = 256, ckpt_interval: int = 0, ckpt_slots=None):
        """prefill() with its scratch in the library's static per-GPU array instead of a workspace."""
        cu, _ = _host_i32(cu_seqlens)
        sl, sl_p = _host_i32(slots)
        hi = np.ascontiguousarray(np.asarray(has_init, dtype=np.uint8))
        _, sp_p = _host_i32(start_pos)
        ns = len(sl)
        max_ck, ck_p = 0, None
        if ckpt_slots is not None:
            ck = np.ascontiguousarray(np.asarray(ckpt_slots, dtype=np.int32).reshape(ns, -1))
            max_ck, ck_p = ck.shape[1], ck.ctypes.data_as(c_void_p)
        xp, xs = _rows(x, "x")
        bp, bs = _rows(B, "B")
        cp, cs = _rows(C, "C")
        zp, zs = _rows(z, "z")
        dp, ds = _rows(dt, "dt")
        yp, ys = _rows(y, "y")
        check(lib().mamba2_prefill_chunked_noalloc(
            self._h, layer, byref(w.struct), ns, cu.ctypes.data_as(c_void_p), sl_p, hi.ctypes.data_as(c_void_p),
            sp_p, xp, xs, bp, bs, cp, cs, zp, zs, dp, ds, _dtype_code(x), yp, ys, _dtype_code(y), chunk_size,
            ckpt_interval, ck_p, max_ck, _stream()))
        return y

    # ------------------------------------------------------------------ checkpoints
    def int8_store(self, num_entries: int) -> "Int8Store":
        """A zeroed int8 checkpoint store of num_entries entries for this pool's layers."""
        return Int8Store(self, num_entries)

    def int8_put(self, store: "Int8Store", layer: int, slots: torch.Tensor, entries: torch.Tensor,
                 slots_host=None, entries_host=None):
        """Quantize slot slots[i] into store entry entries[i] (device int32); layer -1 = all layers."""
        _, s_p = _host_i32(slots_host)
        _, e_p = _host_i32(entries_host)
        check(lib().mamba2_int8_store_put(self._h, byref(store.desc), layer, slots.numel(),
                                          c_void_p(slots.data_ptr()), c_void_p(entries.data_ptr()), s_p, e_p,
                                          _stream()))

    def int8_get(self, store: "Int8Store", layer: int, entries: torch.Tensor, slots: torch.Tensor,
                 entries_host=None, slots_host=None):
        """Restore store entry entries[i] into slot slots[i] (device int32); layer -1 = all layers."""
        _, e_p = _host_i32(entries_host)
        _, s_p = _host_i32(slots_host)
        check(lib().mamba2_int8_store_get(self._h, byref(store.desc), layer, entries.numel(),
                                          c_void_p(entries.data_ptr()), c_void_p(slots.data_ptr()), e_p, s_p,
                                          _stream()))

    def checkpoint(self, layer: int, src: torch.Tensor, dst: torch.Tensor, src_host=None, dst_host=None):
        """Copy both state objects slot src[i] -> dst[i] (device int32); layer -1 = all layers."""
        _, s_p = _host_i32(src_host)
        _, d_p = _host_i32(dst_host)
        check(lib().mamba2_checkpoint_states(self._h, layer, src.numel(), c_void_p(src.data_ptr()),
                                             c_void_p(dst.data_ptr()), s_p, d_p, _stream()))


class Int8Store:
    """int8 checkpoint store for a pool: codes int8 [E, L, H, P, N], scales fp32 [E, L, H, N],
    conv windows [E, L, Cd, W-1] in the pool's conv dtype, allocated on the pool's device."""

    def __init__(self, pool: Pool, num_entries: int):
        cb, sb, vb = c_uint64(), c_uint64(), c_uint64()
        check(lib().mamba2_int8_store_size(pool._h, num_entries, byref(cb), byref(sb), byref(vb)))
        L, H, P, N = pool.num_layers, pool.nheads, pool.head_dim, pool.d_state
        dev = pool.ssm.device
        self.codes = torch.zeros((num_entries, L, H, P, N), dtype=torch.int8, device=dev)
        self.scales = torch.zeros((num_entries, L, H, N), dtype=torch.float32, device=dev)
        self.conv = torch.zeros((num_entries, L) + tuple(pool.conv.shape[2:]), dtype=pool.conv.dtype, device=dev)
        for t, b in ((self.codes, cb), (self.scales, sb), (self.conv, vb)):
            assert t.numel() * t.element_size() == b.value
        self.num_entries = num_entries
        self.desc = Int8StoreDesc(num_entries, 0, self.codes.data_ptr(), self.scales.data_ptr(),
                                  self.conv.data_ptr(), cb.value, sb.value, vb.value)


__all__ = ["Pool", "LayerWeights", "Int8Store", "Mamba2Error"]
