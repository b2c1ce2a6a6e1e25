"""C-ABI checks that run without a GPU.

The library is loaded, every function include/mamba2_pool.h declares must be
exported, the host-only calls (pool_create, pool_info, workspace sizing) are
exercised, and every validation error path is driven with fake device
pointers: validation runs before any HIP call, so none of these calls touches
a device.
"""
import ctypes
import json
import os
import re
import subprocess
import sys
from ctypes import byref, c_uint64, c_void_p

import numpy as np
import pytest

from recurrent_state_update_amd import _ffi
from recurrent_state_update_amd._ffi import Int8StoreDesc, LayerParams, PoolDesc, lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mamba2_pool.h")

ARG, SHAPE, DTYPE, ALIGN, SLOT, UNSUP, HIP, WS = 1, 2, 3, 4, 5, 6, 7, 8
FAKE = 0x7F0000000000          # 256-byte aligned, never dereferenced


def header_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(mamba[12]_\w+)\s*\(", src)))


def test_library_exports_every_declared_function():
    names = header_functions()
    assert len(names) >= 9
    l = lib()
    for n in names:
        assert hasattr(l, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", _ffi.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (mamba[12]_\w+)", out))
    assert set(names) <= exported
    assert set(_ffi.exported_symbols()) == set(names)
    assert l.mamba2_abi_version() == 3


def make_desc(H=128, P=64, N=128, G=8, W=4, L=1, S=4, ssm=1, conv=1, ssm_base=FAKE, conv_base=FAKE):
    es = {0: 4, 1: 2, 2: 2, -1: 2}
    cd = H * P + 2 * G * N
    return PoolDesc(L, S, H, P, N, G, W, ssm, conv, 0, ssm_base, conv_base,
                    L * S * H * P * N * es[ssm], L * S * cd * (W - 1) * es[conv])


def create(desc):
    h = c_void_p()
    st = lib().mamba2_pool_create(byref(desc), byref(h))
    return st, h


@pytest.fixture
def pool():
    st, h = create(make_desc())
    assert st == 0, lib().mamba2_last_error()
    yield h
    lib().mamba2_pool_destroy(h)


def test_pool_info_matches_page_byte_counts():
    g = json.load(open(os.path.join(ROOT, "tests", "golden", "state_sizes.json")))
    by = {e["id"]: e for e in g["entries"]}
    info = {}
    for ssm, conv in ((0, 1), (1, 1)):
        st, h = create(make_desc(ssm=ssm, conv=conv))
        assert st == 0
        a, b = c_uint64(), c_uint64()
        assert lib().mamba2_pool_info(h, byref(a), byref(b)) == 0
        info[(ssm, conv)] = (a.value, b.value)
        lib().mamba2_pool_destroy(h)
    s32, c16 = info[(0, 1)]
    s16, _ = info[(1, 1)]
    assert s16 == 128 * 64 * 128 * 2 == 2 * 2 ** 20
    assert 48 * s16 == by["bf16_ssm_per_layer"]["total_bytes"]
    assert 24 * (s32 + c16) == by["fp32_ssm_bf16_conv_24_layers"]["total_bytes"]
    assert 24 * (s16 + c16) // 131072 == by["bf16_ssm_bf16_conv_24_layers"]["crossover_tokens"]
    assert round((s32 + c16) / 2 ** 20, 2) == by["per_layer_block_mib"]["mib_2dp"]
    assert round(256 * 24 * (s32 + c16) / 2 ** 30, 1) == by["pool_256_slots_gib"]["gib_1dp"]
    assert round(100 * c16 / (s32 + c16), 1) == by["conv_share_percent"]["percent_1dp"]
    assert 2 * s32 == by["long_context_per_layer"]["total_bytes"]


@pytest.mark.parametrize("change,code", [
    (dict(L=0), ARG), (dict(S=0), ARG), (dict(H=0), ARG),
    (dict(H=12, G=8), SHAPE), (dict(P=60), SHAPE), (dict(N=20), SHAPE),
    (dict(W=5), UNSUP), (dict(W=1), UNSUP),
    (dict(ssm=2), DTYPE), (dict(conv=-1), DTYPE),
    (dict(ssm_base=0), ARG), (dict(ssm_base=FAKE + 8), ALIGN), (dict(conv_base=FAKE + 4), ALIGN),
])
def test_pool_create_rejects(change, code):
    st, _ = create(make_desc(**change))
    assert st == code
    assert lib().mamba2_last_error()


def test_pool_create_rejects_wrong_byte_counts():
    d = make_desc()
    d.ssm_bytes += 2
    assert create(d)[0] == SHAPE
    d = make_desc()
    d.conv_bytes -= 16
    assert create(d)[0] == SHAPE


PARAMS = LayerParams(FAKE, FAKE, FAKE, FAKE, FAKE)


def decode(h, **kw):
    a = dict(layer=0, params=byref(PARAMS), batch=2, slots=FAKE, slots_host=None, x=FAKE, xs=8192,
             B=FAKE, Bs=1024, C=FAKE, Cs=1024, z=FAKE, zs=8192, dt=FAKE, dts=128, io=1, y=FAKE, ys=8192, yd=1)
    a.update(kw)
    return lib().mamba2_decode_step(h, a["layer"], a["params"], a["batch"], a["slots"], a["slots_host"],
                                    a["x"], a["xs"], a["B"], a["Bs"], a["C"], a["Cs"], a["z"], a["zs"],
                                    a["dt"], a["dts"], a["io"], a["y"], a["ys"], a["yd"], None)


def test_decode_validation(pool):
    assert decode(pool, batch=0) == 0                     # empty batch: nothing launched
    assert decode(pool, layer=1) == ARG
    assert decode(pool, layer=-1) == ARG
    assert decode(pool, batch=-1) == ARG
    assert decode(pool, params=None) == ARG
    bad = LayerParams(FAKE, 0, FAKE, FAKE, FAKE)
    assert decode(pool, params=byref(bad)) == ARG
    bad = LayerParams(FAKE, FAKE, FAKE, FAKE + 4, FAKE)
    assert decode(pool, params=byref(bad)) == ALIGN
    assert decode(pool, io=3) == DTYPE
    assert decode(pool, yd=7) == DTYPE
    assert decode(pool, slots=None) == ARG
    assert decode(pool, x=None) == ARG
    assert decode(pool, x=FAKE + 2) == ALIGN
    assert decode(pool, xs=8196) == ALIGN
    assert decode(pool, xs=100) == SHAPE
    assert decode(pool, Bs=512) == SHAPE
    assert decode(pool, dts=64) == SHAPE
    assert decode(pool, ys=10) == SHAPE
    sh = (ctypes.c_int32 * 2)(3, 4)
    assert decode(pool, slots_host=sh) == SLOT            # slot 4 of a 4-slot pool
    sh = (ctypes.c_int32 * 2)(2, 2)
    assert decode(pool, slots_host=sh) == SLOT            # duplicate
    sh = (ctypes.c_int32 * 2)(-2, 1)
    assert decode(pool, slots_host=sh) == SLOT
    assert b"slot" in lib().mamba2_last_error()


def test_decode_rejects_unsupported_state_size():
    st, h = create(make_desc(H=8, P=16, N=24, G=1))
    assert st == 0
    assert decode(h, xs=128, Bs=24, Cs=24, zs=128, dts=8, ys=128) == UNSUP
    lib().mamba2_pool_destroy(h)


def test_decode_rejects_a_group_too_wide_for_the_workgroup_lds():
    """The decode workgroup holds its group's x and gate rows in LDS (160 KiB per workgroup): one
    group of 256 heads of 128 rows (32768 per group, 256 KiB) is refused before anything is
    launched; the multi-token decode's per-token share is checked the same way."""
    st, h = create(make_desc(H=256, P=128, N=128, G=1))
    assert st == 0
    assert decode(h, xs=32768, Bs=128, Cs=128, zs=32768, dts=256, ys=32768) == UNSUP
    assert "LDS" in lib().mamba2_last_error().decode()
    lib().mamba2_pool_destroy(h)
    st, h = create(make_desc(H=128, P=64, N=128, G=1))   # 8192 rows: decode fits, 8 tokens do not
    assert st == 0
    assert decode_multi(h, k=8, xs=8192, Bs=128, Cs=128, zs=8192, ys=8192) == UNSUP
    assert "LDS" in lib().mamba2_last_error().decode()
    lib().mamba2_pool_destroy(h)


def prefill(h, cu, slots, has_init=None, start=None, ck=None, max_ck=0, interval=0, chunk=256,
            ws=FAKE, ws_bytes=1 << 40, **kw):
    n = len(slots)
    cu_a = np.asarray(cu, np.int32)
    sl_a = np.asarray(slots, np.int32)
    hi_a = np.asarray(has_init if has_init is not None else [0] * n, np.uint8)
    sp_a = None if start is None else np.asarray(start, np.int32)
    ck_a = None if ck is None else np.asarray(ck, np.int32)
    p = lambda a: None if a is None else a.ctypes.data_as(c_void_p)
    a = dict(x=FAKE, xs=8192, B=FAKE, Bs=1024, C=FAKE, Cs=1024, z=FAKE, zs=8192, dt=FAKE, dts=128, io=1,
             y=FAKE, ys=8192, yd=1, params=byref(PARAMS), layer=0)
    a.update(kw)
    return lib().mamba2_prefill_chunked(h, a["layer"], a["params"], n, p(cu_a), p(sl_a), p(hi_a), p(sp_a),
                                        a["x"], a["xs"], a["B"], a["Bs"], a["C"], a["Cs"], a["z"], a["zs"],
                                        a["dt"], a["dts"], a["io"], a["y"], a["ys"], a["yd"], chunk, interval,
                                        p(ck_a), max_ck, ws, ws_bytes, None)


def test_prefill_validation(pool):
    assert prefill(pool, [0], []) == 0                    # no sequences
    assert prefill(pool, [0, 0, 0], [0, 1]) == 0          # only empty sequences
    assert prefill(pool, [1, 4], [0]) == SHAPE
    assert prefill(pool, [0, 5, 3], [0, 1]) == SHAPE
    assert prefill(pool, [0, 5, 9], [1, 1]) == SLOT
    assert prefill(pool, [0, 5], [4]) == SLOT
    assert prefill(pool, [0, 5], [0], chunk=24) == UNSUP
    assert prefill(pool, [0, 5], [0], chunk=512) == UNSUP
    assert prefill(pool, [0, 5], [0], start=[-1]) == ARG
    ck = [[2, 3]]
    # a checkpoint inside a chunk (position 300 of 600 at chunk 256) ends that chunk: one chunk
    # more than a workspace sized for checkpoints on the chunk grid holds; the library's own size
    # query, given the same host arguments, counts it
    n = wsize(pool, [0, 600])
    assert prefill(pool, [0, 600], [0], ck=ck, max_ck=2, interval=300, ws_bytes=n) == WS
    assert prefill(pool, [0, 600], [0], start=[100], ck=ck, max_ck=2, interval=256, ws_bytes=n) == WS
    n1 = wsize(pool, [0, 600], ck=ck, interval=300)
    assert n1 > n
    assert prefill(pool, [0, 600], [0], ck=ck, max_ck=2, interval=300, ws_bytes=n1 - 1) == WS
    assert wsize(pool, [0, 600], start=[100], ck=ck, interval=256) > n1     # 256 and 512 both inside chunks
    assert wsize(pool, [0, 600], ck=ck, interval=256) == n           # 256 and 512: on the grid
    assert prefill(pool, [0, 600], [0], ck=[[0, 3]], max_ck=2, interval=256) == SLOT  # aliases the slot
    assert prefill(pool, [0, 600], [0], ck=[[2, 2]], max_ck=2, interval=256) == SLOT  # repeated
    assert prefill(pool, [0, 600], [0], ck=[[2, 9]], max_ck=2, interval=256) == SLOT  # range
    assert prefill(pool, [0, 600], [0], ck=None, max_ck=2, interval=256) == ARG
    assert prefill(pool, [0, 5], [0], x=None) == ARG
    assert prefill(pool, [0, 5], [0], zs=100) == SHAPE
    # row strides of x, z and y at or above 16 MiB (bf16: 2^23 elements) are refused
    assert prefill(pool, [0, 5], [0], xs=1 << 23) == SHAPE
    assert prefill(pool, [0, 5], [0], zs=1 << 23) == SHAPE
    assert prefill(pool, [0, 5], [0], ys=1 << 23) == SHAPE
    assert prefill(pool, [0, 5], [0], io=5) == DTYPE
    assert prefill(pool, [0, 5], [0], ws=0) == WS
    assert prefill(pool, [0, 5], [0], ws=FAKE + 128) == WS
    assert prefill(pool, [0, 5], [0], ws_bytes=1024) == WS
    assert prefill(pool, [0, 5], [0], layer=3) == ARG


def wsize(pool, cu, start=None, chunk=256, interval=0, ck=None, expect=0):
    """mamba2_prefill_workspace_size through the C ABI with the call's host arguments."""
    n = c_uint64()
    cu_a = np.asarray(cu, np.int32)
    sp = None if start is None else np.asarray(start, np.int32)
    cka = None if ck is None else np.ascontiguousarray(np.asarray(ck, np.int32))
    st = lib().mamba2_prefill_workspace_size(
        pool, len(cu_a) - 1, cu_a.ctypes.data_as(c_void_p), None if sp is None else sp.ctypes.data_as(c_void_p),
        chunk, interval, None if cka is None else cka.ctypes.data_as(c_void_p), 0 if cka is None else cka.shape[1],
        byref(n))
    assert st == expect, lib().mamba2_last_error()
    return n.value


def test_workspace_size_formula(pool):
    n = c_uint64()
    n.value = wsize(pool, [0, 8192])
    H, P, N, G, T, Q = 128, 64, 128, 8, 8192, 256
    nc = T // Q                                  # the exact chunk count of the call
    planes = 1                                   # bf16 state: single bf16 operand planes
    bc = nc * G * Q * 2 * N * 2 * planes         # post-conv C rows and B columns per (chunk, group)
    vecs = 2 * H * T * 4                         # Delta and its chunk-local cumsum
    cbt = nc * G * 72 * 64 * 8 * 2               # C B^T of the 72 causal (row tile, K-step) pairs, bf16
    total = bc + vecs + cbt
    assert total <= n.value < total + 64 * 1024
    assert n.value < 64 * 1024 * 1024            # fits the static scratch of the no-allocation prefill
    wsize(pool, [0, 8192], chunk=20, expect=UNSUP)
    assert lib().mamba2_prefill_workspace_size(pool, -1, None, None, 256, 0, None, 0, byref(n)) == ARG
    wsize(pool, [1, 8192], expect=SHAPE)
    wsize(pool, [0, 8192, 100], expect=SHAPE)
    wsize(pool, [0, 8192], ck=None, interval=256, expect=0)            # no table: no checkpoints
    assert lib().mamba2_prefill_workspace_size(pool, 1, None, None, 256, 0, None, 0, byref(n)) == ARG
    assert wsize(pool, [0, 0]) == 0


def test_prefill_rejects_unsupported_head_dim():
    st, h = create(make_desc(H=8, P=24, N=16, G=1))
    assert st == 0
    assert prefill(h, [0, 5], [0], xs=192, Bs=16, Cs=16, zs=192, dts=8, ys=192, chunk=16) == UNSUP
    lib().mamba2_pool_destroy(h)


def ckpt(h, src_host, dst_host, layer=0, n=None):
    n = len(src_host) if n is None else n
    s = np.asarray(src_host, np.int32)
    d = np.asarray(dst_host, np.int32)
    return lib().mamba2_checkpoint_states(h, layer, n, FAKE, FAKE, s.ctypes.data_as(c_void_p),
                                          d.ctypes.data_as(c_void_p), None)


def test_checkpoint_validation(pool):
    assert ckpt(pool, [], [], n=0) == 0
    assert ckpt(pool, [0], [1], layer=-2) == ARG
    assert ckpt(pool, [0], [1], layer=1) == ARG
    assert ckpt(pool, [0], [0]) == SLOT
    assert ckpt(pool, [0, 1], [2, 2]) == SLOT
    assert ckpt(pool, [0, 2], [2, 3]) == SLOT        # dst 2 is also a source
    assert ckpt(pool, [0], [4]) == SLOT
    assert ckpt(pool, [-1], [1]) == SLOT
    assert lib().mamba2_checkpoint_states(pool, 0, -1, FAKE, FAKE, None, None, None) == ARG
    assert lib().mamba2_checkpoint_states(pool, 0, 1, None, FAKE, None, None, None) == ARG


def decode_multi(h, **kw):
    a = dict(layer=0, params=byref(PARAMS), batch=2, k=4, si=FAKE, so=FAKE, si_h=None, so_h=None, x=FAKE,
             xs=8192, B=FAKE, Bs=1024, C=FAKE, Cs=1024, z=FAKE, zs=8192, dt=FAKE, dts=128, io=1, y=FAKE, ys=8192,
             yd=1)
    a.update(kw)
    return lib().mamba2_decode_multi(h, a["layer"], a["params"], a["batch"], a["k"], a["si"], a["so"], a["si_h"],
                                     a["so_h"], a["x"], a["xs"], a["B"], a["Bs"], a["C"], a["Cs"], a["z"], a["zs"],
                                     a["dt"], a["dts"], a["io"], a["y"], a["ys"], a["yd"], None)


def test_multi_token_decode_validation(pool):
    i32 = lambda v: (ctypes.c_int32 * len(v))(*v)
    assert decode_multi(pool, batch=0) == 0
    assert decode_multi(pool, k=0) == UNSUP
    assert decode_multi(pool, k=9) == UNSUP
    assert decode_multi(pool, batch=70000) == UNSUP
    assert decode_multi(pool, layer=1) == ARG
    assert decode_multi(pool, si=None) == ARG
    assert decode_multi(pool, so=None) == ARG
    assert decode_multi(pool, io=4) == DTYPE
    assert decode_multi(pool, x=FAKE + 8) == ALIGN
    # host copies (4 slots in the pool): an output that is another row's input, an output twice,
    # an input twice, out of range
    assert decode_multi(pool, k=2, si_h=i32([0, 1]), so_h=i32([2, 1, 3, -1])) == SLOT
    assert decode_multi(pool, k=2, si_h=i32([0, 1]), so_h=i32([2, 3, 3, -1])) == SLOT
    assert decode_multi(pool, k=2, si_h=i32([0, 0]), so_h=i32([2, -1, 3, -1])) == SLOT
    assert decode_multi(pool, k=2, si_h=i32([0, 1]), so_h=i32([2, 9, -1, -1])) == SLOT


def test_mamba1_pool_family():
    """A Mamba1 pool holds a (D, N) state and a (D, W-1) window; the Mamba2 entry points refuse it
    and the Mamba1 decode refuses a Mamba2 pool."""
    D, N, W, S = 64, 16, 4, 4
    d = PoolDesc(1, S, D, 1, N, 1, W, 1, 1, 1, FAKE, FAKE, S * D * N * 2, S * D * (W - 1) * 2)
    st, h = create(d)
    assert st == 0, lib().mamba2_last_error()
    a, b = c_uint64(), c_uint64()
    assert lib().mamba2_pool_info(h, byref(a), byref(b)) == 0
    assert (a.value, b.value) == (D * N * 2, D * (W - 1) * 2)
    wsize(h, [0, 100], chunk=64, expect=UNSUP)
    assert decode(h) == UNSUP
    assert decode_multi(h) == UNSUP
    m1 = lambda hh, **kw: lib().mamba1_decode_step(hh, kw.get("layer", 0), byref(PARAMS), kw.get("batch", 2), FAKE,
                                                  None, FAKE, D, FAKE, N, FAKE, N, FAKE, D, FAKE, D, 1, FAKE, D, 1,
                                                  None)
    assert m1(h, batch=0) == 0
    assert m1(h, layer=1) == ARG
    lib().mamba2_pool_destroy(h)
    st, h2 = create(make_desc())                      # a Mamba2 pool
    assert st == 0
    assert m1(h2, batch=0) == UNSUP
    lib().mamba2_pool_destroy(h2)
    bad = PoolDesc(1, S, D, 2, N, 1, W, 1, 1, 1, FAKE, FAKE, S * D * 2 * N * 2, S * D * 2 * (W - 1) * 2)
    assert create(bad)[0] == SHAPE                    # head_dim must be 1
    bad = PoolDesc(1, S, D, 1, N, 1, W, 1, 1, 7, FAKE, FAKE, S * D * N * 2, S * D * (W - 1) * 2)
    assert create(bad)[0] == ARG                      # unknown family


def store_desc(pool, E=3, **over):
    cb, sb, vb = c_uint64(), c_uint64(), c_uint64()
    assert lib().mamba2_int8_store_size(pool, E, byref(cb), byref(sb), byref(vb)) == 0
    d = dict(num_entries=E, reserved=0, codes=FAKE, scales=FAKE, conv=FAKE, codes_bytes=cb.value,
             scales_bytes=sb.value, conv_bytes=vb.value)
    d.update(over)
    return Int8StoreDesc(**d)


def test_int8_store_sizes_at_the_layer_shape(pool):
    """Dense sizes: codes 1 byte per state element, one fp32 scale per (head, d_state index), the
    conv window at the pool's conv dtype; an entry is about half a bf16 slot."""
    cb, sb, vb = c_uint64(), c_uint64(), c_uint64()
    assert lib().mamba2_int8_store_size(pool, 5, byref(cb), byref(sb), byref(vb)) == 0
    H, P, N, Cd, W = 128, 64, 128, 10240, 4
    assert (cb.value, sb.value, vb.value) == (5 * H * P * N, 5 * H * N * 4, 5 * Cd * (W - 1) * 2)
    ssm, conv = c_uint64(), c_uint64()
    assert lib().mamba2_pool_info(pool, byref(ssm), byref(conv)) == 0
    assert 1.8 < 5 * (ssm.value + conv.value) / (cb.value + sb.value + vb.value) < 2.0
    assert lib().mamba2_int8_store_size(pool, -1, byref(cb), byref(sb), byref(vb)) == ARG


def test_int8_store_validation(pool):
    put, get = lib().mamba2_int8_store_put, lib().mamba2_int8_store_get
    i32 = lambda v: (ctypes.c_int32 * len(v))(*v)
    d = store_desc(pool)
    assert put(pool, byref(d), 0, 0, FAKE, FAKE, None, None, None) == 0      # nothing to do
    assert put(pool, None, 0, 1, FAKE, FAKE, None, None, None) == ARG
    assert put(pool, byref(d), 1, 1, FAKE, FAKE, None, None, None) == ARG   # pool has one layer
    assert put(pool, byref(d), 0, -1, FAKE, FAKE, None, None, None) == ARG
    assert put(pool, byref(d), 0, 1, None, FAKE, None, None, None) == ARG
    bad = store_desc(pool, codes_bytes=d.codes_bytes - 16)
    assert put(pool, byref(bad), 0, 1, FAKE, FAKE, None, None, None) == SHAPE
    bad = store_desc(pool, scales=FAKE + 8)
    assert get(pool, byref(bad), 0, 1, FAKE, FAKE, None, None, None) == ALIGN
    assert put(pool, byref(d), 0, 70000, FAKE, FAKE, None, None, None) == UNSUP
    # host copies: ranges, and distinct destinations (entries for put, slots for get)
    assert put(pool, byref(d), 0, 1, FAKE, FAKE, i32([4]), i32([0]), None) == SLOT    # 4 slots
    assert put(pool, byref(d), 0, 1, FAKE, FAKE, i32([0]), i32([3]), None) == SLOT    # 3 entries
    assert put(pool, byref(d), 0, 2, FAKE, FAKE, i32([0, 1]), i32([2, 2]), None) == SLOT
    assert get(pool, byref(d), 0, 2, FAKE, FAKE, i32([0, 1]), i32([3, 3]), None) == SLOT
    assert get(pool, byref(d), 0, 1, FAKE, FAKE, i32([-1]), i32([0]), None) == SLOT


def test_last_error_is_cleared_by_success(pool):
    assert decode(pool, layer=5) == ARG
    assert lib().mamba2_last_error() != b""
    a, b = c_uint64(), c_uint64()
    assert lib().mamba2_pool_info(pool, byref(a), byref(b)) == 0
    assert lib().mamba2_last_error() == b""


def test_destroy_null_is_noop():
    lib().mamba2_pool_destroy(None)


def test_mamba1_prefill_validation():
    """Mamba1 prefill: sizing, family, slot, shape and workspace errors, all raised on the host
    before any device work (the too-small workspace is the last check before the table upload)."""
    D, N, W, S = 64, 16, 4, 6
    i32 = lambda v: np.ascontiguousarray(np.asarray(v, dtype=np.int32))
    st, h = create(PoolDesc(1, S, D, 1, N, 1, W, 1, 1, 1, FAKE, FAKE, S * D * N * 2, S * D * (W - 1) * 2))
    assert st == 0, lib().mamba2_last_error()
    n0, n1, n2 = c_uint64(), c_uint64(), c_uint64()
    assert lib().mamba1_prefill_workspace_size(h, 2, 100, 32, 0, byref(n0)) == 0
    assert lib().mamba1_prefill_workspace_size(h, 2, 1000, 32, 0, byref(n1)) == 0
    assert lib().mamba1_prefill_workspace_size(h, 2, 1000, 32, 4, byref(n2)) == 0
    # end state and entering state per chunk (2 x D N fp32) dominate the growth
    assert n1.value - n0.value >= (1000 // 32 - 100 // 32) * 2 * D * N * 4
    assert n2.value >= n1.value and n0.value % 256 == 0
    assert lib().mamba1_prefill_workspace_size(h, 2, 100, 8, 0, byref(n0)) == UNSUP
    # chunk_size 0: the library chooses; at D 64 two sequences give 2 workgroups per chunk, far
    # from filling the GPU, so the rows are cut into 16-row chunks
    n3, n4 = c_uint64(), c_uint64()
    assert lib().mamba1_prefill_workspace_size(h, 2, 100, 0, 0, byref(n3)) == 0
    assert lib().mamba1_prefill_workspace_size(h, 2, 100, 16, 0, byref(n4)) == 0
    assert n3.value == n4.value
    # a size taken for more rows serves fewer (the chunk count bound only grows with the rows)
    for t in (100, 200, 1000, 50000):
        a_, b_ = c_uint64(), c_uint64()
        assert lib().mamba1_prefill_workspace_size(h, 2, t, 0, 0, byref(a_)) == 0
        assert lib().mamba1_prefill_workspace_size(h, 2, t + 37, 0, 0, byref(b_)) == 0
        assert b_.value >= a_.value
    wsize(h, [0, 50, 100], chunk=64, expect=UNSUP)

    def call(hh=None, **kw):
        cu = i32(kw.get("cu", [0, 40, 100]))
        sl = i32(kw.get("slots", [0, 1]))
        hi = np.asarray(kw.get("has_init", [1, 0]), dtype=np.uint8)
        ck = kw.get("ck")
        ck_p = ck.ctypes.data_as(c_void_p) if ck is not None else None
        return lib().mamba1_prefill(
            hh or h, kw.get("layer", 0), byref(PARAMS), len(sl), cu.ctypes.data_as(c_void_p),
            sl.ctypes.data_as(c_void_p), hi.ctypes.data_as(c_void_p), None, FAKE, D, kw.get("B", FAKE),
            kw.get("Bs", N), FAKE, N, FAKE, D, FAKE, D, 1, FAKE, D, 1, kw.get("chunk", 32),
            kw.get("interval", 0), ck_p, ck.shape[1] if ck is not None else 0, kw.get("ws", FAKE),
            kw.get("ws_bytes", 64), None)

    assert call() == WS                                   # 64 bytes is far too small
    assert call(ws=FAKE + 16, ws_bytes=1 << 40) == WS     # misaligned
    assert call(cu=[0, 0, 0]) == 0                        # no rows: nothing to do
    assert call(layer=1) == ARG
    assert call(chunk=8) == UNSUP
    assert call(chunk=4097) == UNSUP
    assert call(chunk=0) == WS                            # the library's choice is valid
    assert call(slots=[0, 0]) == SLOT
    assert call(slots=[0, 6]) == SLOT
    assert call(cu=[0, 50, 40]) == SHAPE
    assert call(cu=[1, 50, 60]) == SHAPE
    assert call(B=FAKE + 4) == ALIGN
    assert call(Bs=N + 2) == ALIGN
    assert call(interval=16, ck=i32([[2, 3], [1, -1]])) == SLOT     # aliases sequence 1's slot
    assert call(interval=16, ck=i32([[2, 3], [3, -1]])) == SLOT     # repeats
    assert call(interval=16, ck=i32([[2, 3], [4, -1]])) == WS       # valid up to the workspace
    st, h2 = create(make_desc())
    assert st == 0
    assert call(h2) == UNSUP                                         # a Mamba2 pool
    lib().mamba2_pool_destroy(h2)
    lib().mamba2_pool_destroy(h)


def test_header_is_plain_c_and_links_against_the_library(tmp_path):
    """include/mamba2_pool.h compiles as C99 (no C++ in the ABI), and a C program that calls the
    host-only entry points through it links against libmamba2pool.so and runs without a GPU."""
    prog = tmp_path / "abi.c"
    prog.write_text(r'''
#include <stdio.h>
#include <string.h>
#include "mamba2_pool.h"
int main(void) {
  if (mamba2_abi_version() != 3) return 1;
  m2_pool_desc d;
  memset(&d, 0, sizeof d);
  d.num_layers = 1; d.num_slots = 2; d.nheads = 4; d.head_dim = 8; d.d_state = 16; d.n_groups = 1;
  d.conv_kernel = 4; d.ssm_dtype = M2_BF16; d.conv_dtype = M2_BF16;
  d.ssm_base = (void*)0x7F0000000000ull; d.conv_base = (void*)0x7F0000000000ull;
  d.ssm_bytes = 1ull * 2 * 4 * 8 * 16 * 2; d.conv_bytes = 1ull * 2 * (4 * 8 + 2 * 16) * 3 * 2;
  m2_pool* p = 0;
  if (mamba2_pool_create(&d, &p) != M2_OK) { printf("%s\n", mamba2_last_error()); return 2; }
  uint64_t s = 0, c = 0;
  if (mamba2_pool_info(p, &s, &c) != M2_OK || s != 4 * 8 * 16 * 2 || c != 64 * 3 * 2) return 3;
  d.nheads = 3;                                          /* not a multiple of n_groups = 2 below */
  d.n_groups = 2;
  m2_pool* q = 0;
  if (mamba2_pool_create(&d, &q) == M2_OK || strlen(mamba2_last_error()) == 0) return 4;
  /* workspace of a 600-row prefill at chunk 256, without and with checkpoints at 300 and 600:
     the one at 300 ends a chunk early, and the library counts it from the same host arguments */
  int32_t cu[2] = {0, 600}, ck[2] = {1, -1};
  uint64_t w0 = 0, w1 = 0, w2 = 0;
  if (mamba2_prefill_workspace_size(p, 1, cu, NULL, 256, 0, NULL, 0, &w0) != M2_OK || w0 == 0) return 5;
  if (mamba2_prefill_workspace_size(p, 1, cu, NULL, 256, 300, ck, 2, &w1) != M2_OK || w1 <= w0) return 6;
  if (mamba2_prefill_workspace_size(p, 1, cu, NULL, 256, 512, ck, 2, &w2) != M2_OK || w2 >= w1) return 7;
  mamba2_pool_destroy(p);
  printf("ok\n");
  return 0;
}
''')
    exe = tmp_path / "abi"
    lib_dir = os.path.dirname(_ffi.LIB_PATH)
    r = subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"), str(prog),
                        "-L", lib_dir, "-lmamba2pool", f"-Wl,-rpath,{lib_dir}", "-o", str(exe)],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0 and r.stdout.strip() == "ok", (r.returncode, r.stdout, r.stderr)


def test_binding_fails_loudly_without_the_library(tmp_path):
    """With the shared library absent the binding raises instead of falling back to anything: run
    in a fresh interpreter whose library path points at a file that does not exist."""
    code = ("import sys; sys.path.insert(0, %r)\n"
            "from recurrent_state_update_amd import _ffi\n"
            "_ffi.LIB_PATH = %r\n"
            "try:\n"
            "    _ffi.lib()\n"
            "except RuntimeError as e:\n"
            "    print('raised:', e)\n"
            "else:\n"
            "    print('loaded')\n") % (ROOT, str(tmp_path / "missing.so"))
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    assert r.stdout.startswith("raised:") and "not built" in r.stdout


# ---- GDN and KDA pools: state only (the pages give no recurrence for either)
FAMILY_CODE = {"Mamba2": 0, "Mamba1": 1, "GDN": 2, "KDA": 3}
DT_CODE = {"fp32": 0, "bf16": 1}


def mambaspec():
    return json.load(open(os.path.join(ROOT, "tests", "golden", "mambaspec_state_shapes.json")))


def family_desc(family, dims, W=4, L=2, S=5):
    """A descriptor built from the table's symbols: recurrent shape and dtypes from the MambaSpec
    entry, the conv channel count D of the q, k, v projections (GDN: 2 Hk dk + Hv dv; KDA: 3 H d)."""
    spec = mambaspec()
    f = spec["families"][family]
    rec = [dims[k] for k in f["recurrent"]]
    conv_dt, ssm_dt = f["dtypes"]
    by = spec["dtype_bytes"]
    if family == "GDN":
        H, P, N, G = dims["num_v_heads"], dims["head_v_dim"], dims["head_k_dim"], dims["num_k_heads"]
        D = 2 * G * N + H * P
    else:
        H, P, N, G = dims["num_heads"], dims["head_dim"], dims["head_dim"], dims["num_heads"]
        D = 3 * H * P
    rec_bytes = int(np.prod(rec)) * by[ssm_dt]
    conv_bytes = D * (W - 1) * by[conv_dt]
    d = PoolDesc(L, S, H, P, N, G, W, DT_CODE[ssm_dt], DT_CODE[conv_dt], FAMILY_CODE[family], FAKE, FAKE,
                 L * S * rec_bytes, L * S * conv_bytes)
    return d, rec_bytes, conv_bytes


GDN_DIMS = [dict(num_v_heads=32, head_v_dim=128, head_k_dim=128, num_k_heads=16),
            dict(num_v_heads=8, head_v_dim=64, head_k_dim=32, num_k_heads=2)]
KDA_DIMS = [dict(num_heads=32, head_dim=128), dict(num_heads=4, head_dim=64)]


@pytest.mark.parametrize("family,dims", [("GDN", d) for d in GDN_DIMS] + [("KDA", d) for d in KDA_DIMS])
def test_gdn_and_kda_pools_hold_the_table_byte_counts(family, dims):
    """pool_info of a GDN or KDA pool equals the MambaSpec table's recurrent shape times its dtype
    size, and the conv window D x (kernel-1) at the conv dtype; the int8 store of such a pool has
    one code per state element and one fp32 scale per (head, last state index)."""
    d, rec_bytes, conv_bytes = family_desc(family, dims)
    st, h = create(d)
    assert st == 0, lib().mamba2_last_error()
    a, b = c_uint64(), c_uint64()
    assert lib().mamba2_pool_info(h, byref(a), byref(b)) == 0
    assert (a.value, b.value) == (rec_bytes, conv_bytes)
    cb, sb, vb = c_uint64(), c_uint64(), c_uint64()
    assert lib().mamba2_int8_store_size(h, 3, byref(cb), byref(sb), byref(vb)) == 0
    L = d.num_layers
    assert cb.value == 3 * L * d.nheads * d.head_dim * d.d_state
    assert sb.value == 3 * L * d.nheads * d.d_state * 4
    assert vb.value == 3 * L * conv_bytes
    lib().mamba2_pool_destroy(h)


def test_gdn_and_kda_byte_counts_at_their_published_widths():
    """The two wide configurations above by hand: a GDN layer with 32 value heads of 128 x 128
    holds 1 MiB of bf16 state; a KDA layer with 32 heads of 128 x 128 holds 2 MiB of fp32 state."""
    for family, dims, rec in (("GDN", GDN_DIMS[0], 32 * 128 * 128 * 2), ("KDA", KDA_DIMS[0], 32 * 128 * 128 * 4)):
        d, rec_bytes, conv_bytes = family_desc(family, dims)
        assert rec_bytes == rec
        st, h = create(d)
        assert st == 0
        a, b = c_uint64(), c_uint64()
        assert lib().mamba2_pool_info(h, byref(a), byref(b)) == 0 and a.value == rec
        lib().mamba2_pool_destroy(h)


def test_gdn_and_kda_pools_are_validated_and_refused_by_the_recurrences():
    d, _, _ = family_desc("KDA", KDA_DIMS[1])
    st, h = create(d)
    assert st == 0, lib().mamba2_last_error()
    assert decode(h) == UNSUP
    assert decode_multi(h) == UNSUP
    assert prefill(h, [0, 16], [0]) == UNSUP
    wsize(h, [0, 100], chunk=64, expect=UNSUP)
    n = c_uint64()
    assert lib().mamba1_prefill_workspace_size(h, 2, 100, 32, 0, byref(n)) == UNSUP
    assert ckpt(h, [0], [5]) == SLOT                # the copy validates any family (it runs on the GPU tests)
    lib().mamba2_pool_destroy(h)
    # KDA: square state per head, n_groups = nheads, conv bf16 + state fp32
    H, P, W, L, S = 4, 64, 4, 2, 5
    kda = lambda P, N, G, ssm, conv: PoolDesc(L, S, H, P, N, G, W, ssm, conv, 3, FAKE, FAKE,
                                              L * S * H * P * N * (4 if ssm == 0 else 2),
                                              L * S * (H * P + 2 * G * N) * (W - 1) * (4 if conv == 0 else 2))
    assert create(kda(P, 32, H, 0, 1))[0] == SHAPE          # head_dim != d_state
    assert create(kda(P, P, 2, 0, 1))[0] == SHAPE           # n_groups != nheads
    assert create(kda(P, P, H, 1, 1))[0] == DTYPE           # bf16 state
    assert create(kda(P, P, H, 0, 0))[0] == DTYPE           # fp32 conv
    assert create(kda(P, P, H, 0, 1))[0] == 0
    # GDN: value heads a multiple of key heads, both objects bf16
    gdn = lambda H, G, ssm: PoolDesc(L, S, H, 64, 32, G, W, ssm, 1, 2, FAKE, FAKE,
                                     L * S * H * 64 * 32 * (4 if ssm == 0 else 2), L * S * (H * 64 + 2 * G * 32) * (W - 1) * 2)
    assert create(gdn(6, 4, 1))[0] == SHAPE                 # 6 value heads over 4 key heads
    assert create(gdn(8, 2, 0))[0] == DTYPE                 # fp32 state
    assert create(gdn(8, 2, 1))[0] == 0
    bad = PoolDesc(L, S, H, 1, 16, 1, W, 1, 1, 4, FAKE, FAKE, L * S * H * 16 * 2, L * S * H * (W - 1) * 2)
    assert create(bad)[0] == ARG                            # no family 4
