"""CPU oracle for the Mamba2 selective-state update over a slot pool (fp64).

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only the test suite, the smoke check
of the package entry point and the benchmark's CPU-baseline leg may import
this module.  The HIP library never calls it, and this module imports nothing
from the HIP side.

What it computes, and where the pages say so
--------------------------------------------
Sources are four web pages on hybrid-model recurrent state:
 * "Hybrid SSM / Mamba models and non-KV state" (mlinterviewnotes.com, ch. 7.3),
   cited below as [SSM-hybrids];
 * "hybrid-attn-ssm-kv-cache-sizing" (phantomic12.github.io), [sizing];
 * "Hybrid KV cache vs recurrent state memory" (fanout.sh), [fanout];
 * Mamba study notes (echobase-5bl.pages.dev, 2026.07.27.01), [notes].

Per token t, per head h of group g = h // (H/G) (contiguous head->group map):
 1. conv: a rolling window of the last W-1 raw inputs per channel ([SSM-hybrids],
    the passage on the two state objects: the short-convolution state has shape
    (d_conv, W-1), d_conv = d_inner + 2*g*d_state), extended by the current
    input u_t, feeds a causal depthwise Conv1d with bias, then SiLU
    ([notes], "Mamba": x = SiLU(Conv1d(x'))).  All d_conv channels pass the
    conv, in the order [x (H*P) | B (G*N) | C (G*N)].
 2. Delta = softplus(dt + dt_bias) ([SSM-hybrids], the decode call with
    dt_bias and dt_softplus=True; [notes] Delta_t = Softplus(...)).
 3. h_t = exp(Delta*A) h_{t-1} + Delta * x_t B_t^T      ([notes], "Mamba")
 4. y_t = h_t C_t + D x_t   (readout of the new state; [notes], classic SSM
    output y = C h + D x, and the Mamba readout y_t = C_t h_t)
 5. out_t = y_t * SiLU(z_t)                              ([notes], "Mamba")
State lives in slots of a pool indexed [layer, slot, ...], one dense tensor
per state object ([SSM-hybrids], MambaPool passage); the temporal state
has shape (H, P, N) ([SSM-hybrids], the state-shape function).

Readings where the pages are silent (each also listed in the design notes):
 * A is one negative scalar per head, passed directly; B-bar = Delta*B.
 * conv tap k = W-1 multiplies the current token (causal cross-correlation).
 * softplus is log(1 + e^v) evaluated exactly (no threshold).
 * Stored state is rounded to its storage dtype: fp64 -> fp32 (RNE) -> bf16
   (RNE on the fp32 bit pattern).  Decode rounds after every step; prefill
   keeps the running state in fp64 and rounds only what it stores (final
   state and checkpoints).  y is rounded to its output dtype.
 * The conv window holds raw inputs rounded to the conv dtype; inside one
   prefill call the conv reads the call's own inputs unrounded.
 * has_initial_state = 0 means a zero state and a zero window; the slot is not read.
 * A checkpoint at absolute position p (start_pos < p <= start_pos + L,
   p % interval == 0) stores round(state after p tokens) and the window of the
   raw inputs at positions p-W+1 .. p-1.

Checkpoints may also be held in an int8 store apart from the pool ([SSM-hybrids],
SGLang int8 checkpoint passage): see int8_quantize below for the arithmetic.
Several decode tokens per sequence with a snapshot after each (speculative decode):
decode_multi.  A second recurrent family on the same kind of pool, Mamba1 with a (D, N)
state: Mamba1PoolRef, mamba1_decode_step and mamba1_prefill (the same token recurrence
over packed sequences with the prefill's rounding and checkpoint rules).

Parity pins live in the test suite (matrix form of [notes] "Mamba and
Attention", constant-input closed form, scipy lfilter scalar case,
np.convolve conv, torch bf16 casts, byte counts printed on the pages; for the
int8 store: states built from known codes and power-of-two scales, halves
rounding to even, the half-step error bound, the page's ~2x capacity, and the
restored error evolving through the decay product; for multi-token decode: a prefill
that checkpoints after every token; for Mamba1: equality with the Mamba2 step when
the decay does not depend on the state index, the constant-input closed form, and a
prefill equal to its rows as decode steps with an initial-state perturbation evolving
through the product of the decays).
"""
from __future__ import annotations

import numpy as np

_BYTES = {"f64": 8, "f32": 4, "bf16": 2}


# --------------------------------------------------------------------------
# rounding to a storage dtype
# --------------------------------------------------------------------------
def round_to(x, dtype: str) -> np.ndarray:
    """Round float64 values to ``dtype`` and return them as float64.

    'f64' is the identity, 'f32' is numpy's round-to-nearest-even cast, and
    'bf16' rounds the fp32 bit pattern to its upper 16 bits with ties to even
    (NaN stays a quiet NaN, overflow goes to infinity).
    """
    x = np.asarray(x, dtype=np.float64)
    if dtype == "f64":
        return x.copy()
    with np.errstate(over="ignore", invalid="ignore"):
        x32 = x.astype(np.float32)
    if dtype == "f32":
        return x32.astype(np.float64)
    if dtype != "bf16":
        raise ValueError(dtype)
    bits = x32.view(np.uint32)
    lsb = (bits >> np.uint32(16)) & np.uint32(1)
    # uint32 arithmetic: only NaN bit patterns can wrap, and NaN takes the other branch
    with np.errstate(over="ignore"):
        rounded = (bits + np.uint32(0x7FFF) + lsb) & np.uint32(0xFFFF0000)
    quiet = (bits | np.uint32(0x00400000)) & np.uint32(0xFFFF0000)
    out = np.where(np.isnan(x32), quiet, rounded).astype(np.uint32)
    return out.view(np.float32).astype(np.float64)


# --------------------------------------------------------------------------
# elementwise functions
# --------------------------------------------------------------------------
def silu(v):
    """SiLU(v) = v / (1 + e^-v)."""
    v = np.asarray(v, dtype=np.float64)
    with np.errstate(over="ignore"):
        return v / (1.0 + np.exp(-v))


def softplus(v):
    """softplus(v) = log(1 + e^v), written as max(v, 0) + log1p(e^-|v|)."""
    v = np.asarray(v, dtype=np.float64)
    return np.maximum(v, 0.0) + np.log1p(np.exp(-np.abs(v)))


# --------------------------------------------------------------------------
# the two state objects of a slot pool
# --------------------------------------------------------------------------
class PoolRef:
    """Oracle copy of a slot pool: ssm[layer, slot, H, P, N], conv[layer, slot, Cd, W-1].

    Values are float64 holding numbers representable in the storage dtypes.
    Slots the oracle never writes keep whatever the caller put there.
    """

    def __init__(self, shape, num_layers: int, num_slots: int, ssm_dtype: str, conv_dtype: str):
        H, P, N = shape.nheads, shape.head_dim, shape.d_state
        self.shape = shape
        self.ssm_dtype, self.conv_dtype = ssm_dtype, conv_dtype
        self.ssm = np.zeros((num_layers, num_slots, H, P, N))
        self.conv = np.zeros((num_layers, num_slots, shape.conv_dim, shape.conv_kernel - 1))

    def ssm_bytes_per_slot_layer(self) -> int:
        """Temporal state bytes of one slot in one layer: H * P * N * sizeof(dtype)."""
        s = self.shape
        return s.nheads * s.head_dim * s.d_state * _BYTES[self.ssm_dtype]

    def conv_bytes_per_slot_layer(self) -> int:
        """Conv window bytes of one slot in one layer: d_conv * (W - 1) * sizeof(dtype)."""
        s = self.shape
        return s.conv_dim * (s.conv_kernel - 1) * _BYTES[self.conv_dtype]


def _f64(a) -> np.ndarray:
    """Inputs arrive as exact values of their storage dtype; lift them to fp64."""
    return np.asarray(a, dtype=np.float64)


def _split(act, shape):
    """Post-conv activations (..., Cd) -> x (..., H, P), B (..., G, N), C (..., G, N)."""
    I, G, N = shape.intermediate, shape.n_groups, shape.d_state
    lead = act.shape[:-1]
    x = act[..., :I].reshape(lead + (shape.nheads, shape.head_dim))
    B = act[..., I:I + G * N].reshape(lead + (G, N))
    C = act[..., I + G * N:].reshape(lead + (G, N))
    return x, B, C


# --------------------------------------------------------------------------
# decode: one token per sequence, in place on the pool
# --------------------------------------------------------------------------
def decode_step(pool: PoolRef, layer: int, params: dict, slots, u, z, dt, y_dtype: str):
    """One decode token for each batch row.  Returns out (batch, H*P), rounded to y_dtype.

    slots[b] < 0 is a padding row: the pool is neither read nor written and
    its output row is zero.
    """
    s = pool.shape
    H, P, G = s.nheads, s.head_dim, s.n_groups
    hpg = H // G
    gidx = np.arange(H) // hpg
    A, D, dt_bias, w, b = (_f64(params[k]) for k in ("A", "D", "dt_bias", "conv_w", "conv_b"))
    out = np.zeros((len(slots), s.intermediate))
    for r, slot in enumerate(slots):
        if slot < 0:
            continue
        window = np.concatenate([pool.conv[layer, slot], _f64(u[r])[:, None]], axis=1)
        act = silu(b + np.sum(w * window, axis=1))                     # step 1
        x, Bm, Cm = _split(act, s)
        delta = softplus(_f64(dt[r]) + dt_bias)                        # step 2
        alpha = np.exp(delta * A)
        h = pool.ssm[layer, slot]
        h_new = alpha[:, None, None] * h + (delta[:, None] * x)[:, :, None] * Bm[gidx][:, None, :]   # 3
        y = np.einsum("hpn,hn->hp", h_new, Cm[gidx]) + D[:, None] * x  # step 4
        out[r] = (y.reshape(-1)) * silu(_f64(z[r]))                    # step 5
        pool.ssm[layer, slot] = round_to(h_new, pool.ssm_dtype)
        pool.conv[layer, slot] = round_to(window[:, 1:], pool.conv_dtype)
    return round_to(out, y_dtype)


# --------------------------------------------------------------------------
# the selective scan on post-conv inputs (one head)
# --------------------------------------------------------------------------
def ssm_scan(h0, x, Bm, Cm, delta, A: float, D: float):
    """Token-by-token recurrence for one head; returns (y before the gate, final state).

    h0 (P, N); x (L, P); Bm, Cm (L, N); delta (L,).
    """
    h = np.array(h0, dtype=np.float64, copy=True)
    x, Bm, Cm, delta = _f64(x), _f64(Bm), _f64(Cm), _f64(delta)
    y = np.zeros_like(x)
    for t in range(len(delta)):
        h = np.exp(delta[t] * A) * h + delta[t] * np.outer(x[t], Bm[t])
        y[t] = h @ Cm[t] + D * x[t]
    return y, h


def ssd_matrix_form(h0, x, Bm, Cm, delta, A: float, D: float):
    """The semiseparable form Y = (M o L) X of [notes] ("Mamba and Attention"), one head.

    M[i, j] = C_i . (prod_{k=j+1..i} Abar_k) Bbar_j with Abar_k = exp(Delta_k A)
    and Bbar_j = Delta_j B_j; L is the causal mask.  A nonzero initial state
    adds (prod_{k<=i} Abar_k) C_i . h0[p, :] to row i.  Built element by
    element from the products, with no cumulative sums.
    """
    L = len(delta)
    x, Bm, Cm, delta, h0 = _f64(x), _f64(Bm), _f64(Cm), _f64(delta), _f64(h0)
    abar = np.exp(delta * A)
    M = np.zeros((L, L))
    for i in range(L):
        for j in range(i + 1):
            M[i, j] = (Cm[i] @ Bm[j]) * np.prod(abar[j + 1:i + 1]) * delta[j]
    init = np.array([np.prod(abar[:i + 1]) * (np.asarray(h0) @ Cm[i]) for i in range(L)])
    return M @ x + D * np.asarray(x) + init


def decode_multi(pool: PoolRef, layer: int, params: dict, slots_in, slots_out, u, z, dt, y_dtype: str):
    """Several decode tokens per sequence (a verified token and its drafts), with the state after
    every token kept in a slot of its own ([SSM-hybrids]: the conv state widened by num_spec and
    one extra state block per speculative token, so that the state at whichever token the
    verifier accepts is at hand).

    Row b starts from slot slots_in[b]; its K tokens u[b, t] (t = 0..K-1) are decode steps in
    order, each rounding the state it stores as decode does; the state and window after token t
    go to slot slots_out[b][t] (< 0: not kept).  slots_in itself is left as it was unless it is
    also an output slot.  Returns out (batch, K, H*P); a padding row (slots_in[b] < 0) reads and
    writes nothing and its outputs are zero.
    """
    s = pool.shape
    batch, K = len(slots_in), np.asarray(u).shape[1]
    out = np.zeros((batch, K, s.intermediate))
    for r, slot in enumerate(slots_in):
        if slot < 0:
            continue
        work = PoolRef(s, 1, 1, pool.ssm_dtype, pool.conv_dtype)
        work.ssm[0, 0], work.conv[0, 0] = pool.ssm[layer, slot], pool.conv[layer, slot]
        snaps = []
        for t in range(K):
            out[r, t] = decode_step(work, 0, params, [0], np.asarray(u)[r, t:t + 1], np.asarray(z)[r, t:t + 1],
                                    np.asarray(dt)[r, t:t + 1], y_dtype)[0]
            snaps.append((work.ssm[0, 0].copy(), work.conv[0, 0].copy()))
        for t, o in enumerate(slots_out[r]):
            if o >= 0:
                pool.ssm[layer, o], pool.conv[layer, o] = snaps[t]
    return out


# --------------------------------------------------------------------------
# prefill: packed variable-length sequences, chunk boundaries are invisible
# --------------------------------------------------------------------------
def conv_tokens(window0, u, conv_w, conv_b):
    """Causal depthwise conv over a token stream: (W-1, C) initial window rows + (L, C) inputs.

    Returns pre-activation v (L, C): v[t, c] = b[c] + sum_k w[c, k] * stream[t + k, c].
    """
    stream = np.concatenate([_f64(window0), _f64(u)], axis=0)
    conv_w, conv_b = _f64(conv_w), _f64(conv_b)
    W = conv_w.shape[1]
    L = u.shape[0]
    v = np.broadcast_to(conv_b, (L, conv_b.shape[0])).copy()
    for k in range(W):
        v += conv_w[:, k] * stream[k:k + L]
    return v


def prefill(pool: PoolRef, layer: int, params: dict, cu_seqlens, slots, has_init, start_pos,
            u, z, dt, y_dtype: str, ckpt_interval: int = 0, ckpt_slots=None, heads=None):
    """Prefill packed sequences (cu_seqlens) into their slots; returns out (T, H*P).

    heads (optional) restricts the recurrence and the state writes to those
    heads; output columns of other heads are NaN.  Conv windows are always
    written in full.  Checkpoints follow the rule in the module docstring.
    """
    s = pool.shape
    H, P, N, G, W, I = s.nheads, s.head_dim, s.d_state, s.n_groups, s.conv_kernel, s.intermediate
    heads = np.arange(H) if heads is None else np.asarray(heads, dtype=np.int64)
    hpg = H // G
    groups = heads // hpg
    ug = np.unique(groups)
    # channels this call needs: x of the chosen heads, B and C of their groups
    xch = (heads[:, None] * P + np.arange(P)).ravel()
    bch = (I + ug[:, None] * N + np.arange(N)).ravel()
    cch = (I + G * N + ug[:, None] * N + np.arange(N)).ravel()
    chans = np.concatenate([xch, bch, cch])
    gpos = {g: i for i, g in enumerate(ug)}
    gsel = np.array([gpos[g] for g in groups])
    A, D, dt_bias = (_f64(params[k])[heads] for k in ("A", "D", "dt_bias"))
    T = int(cu_seqlens[-1])
    outs = np.zeros((T, len(heads), P))                          # outputs of the chosen heads
    for sq in range(len(slots)):
        t0, t1 = int(cu_seqlens[sq]), int(cu_seqlens[sq + 1])
        L = t1 - t0
        if L == 0:
            continue
        slot = int(slots[sq])
        if has_init[sq]:
            h = pool.ssm[layer, slot][heads].copy()
            win0 = pool.conv[layer, slot].T.copy()                 # (W-1, Cd)
        else:
            h = np.zeros((len(heads), P, N))
            win0 = np.zeros((W - 1, s.conv_dim))
        useq = _f64(u[t0:t1])
        stream = np.concatenate([win0, useq], axis=0)             # raw inputs, window first
        act = silu(conv_tokens(win0[:, chans], useq[:, chans],
                               params["conv_w"][chans], params["conv_b"][chans]))
        nx = len(xch)
        x = act[:, :nx].reshape(L, len(heads), P)
        Bm = act[:, nx:nx + len(bch)].reshape(L, len(ug), N)[:, gsel]
        Cm = act[:, nx + len(bch):].reshape(L, len(ug), N)[:, gsel]
        delta = softplus(_f64(dt[t0:t1])[:, heads] + dt_bias)
        alpha = np.exp(delta * A)
        zs = silu(_f64(z[t0:t1]).reshape(L, H, P)[:, heads])
        sp = int(start_pos[sq])
        for t in range(L):
            h = alpha[t][:, None, None] * h + (delta[t][:, None] * x[t])[:, :, None] * Bm[t][:, None, :]
            y = np.einsum("hpn,hn->hp", h, Cm[t]) + D[:, None] * x[t]
            outs[t0 + t] = y * zs[t]
            p = sp + t + 1
            if ckpt_interval and p % ckpt_interval == 0:
                k = p // ckpt_interval - sp // ckpt_interval - 1
                dst = int(ckpt_slots[sq][k]) if k < len(ckpt_slots[sq]) else -1
                if dst >= 0:
                    pool.ssm[layer, dst][heads] = round_to(h, pool.ssm_dtype)
                    pool.conv[layer, dst] = round_to(stream[t + 1:t + W].T, pool.conv_dtype)
        pool.ssm[layer, slot][heads] = round_to(h, pool.ssm_dtype)
        pool.conv[layer, slot] = round_to(stream[L:L + W - 1].T, pool.conv_dtype)
    out = np.full((T, H, P), np.nan)
    out[:, heads] = round_to(outs, y_dtype)
    return out.reshape(T, I)


# --------------------------------------------------------------------------
# int8 checkpoint store
# --------------------------------------------------------------------------
# [SSM-hybrids], the SGLang passage on compressed checkpoints: cached states are
# kept apart from the active pool, the temporal state in int8 with symmetric
# scales per (head, k-channel), quantized once when stored and dequantized once
# into a fresh active slot on a prefix hit; the conv window stays in its own
# dtype.  Reading taken for the k-channel: the d_state index n (B is the key
# the state is written with, h += Delta x B^T), so one scale covers the head_dim
# entries h[h, :, n].  The pages fix neither the rounding nor the arithmetic;
# both here are fp32, the precision of the kernels, so that the integer codes
# are decided the same way on both sides:
#     amax = max_p |h[h, p, n]|      scale = fp32(amax / 127)
#     inv  = fp32(127 / amax)        code  = clamp(rint(fp32(h * inv)), -127, 127)
#     restored = round_to(fp32(code * scale), ssm dtype)
# A column of zeros gets scale 0 and codes 0.

def int8_quantize(state) -> tuple[np.ndarray, np.ndarray]:
    """Codes (int8, same shape) and scales (fp32, the head_dim axis -2 reduced) of a temporal
    state [..., H, P, N] holding values of its fp32 or bf16 storage dtype."""
    s32 = np.asarray(state, np.float64).astype(np.float32)
    amax = np.max(np.abs(s32), axis=-2)
    with np.errstate(divide="ignore"):
        scale = (amax / np.float32(127.0)).astype(np.float32)
        inv = np.where(amax > 0, np.float32(127.0) / amax, np.float32(0.0)).astype(np.float32)
    prod = (s32 * inv[..., None, :]).astype(np.float32)
    codes = np.clip(np.rint(prod), -127, 127).astype(np.int8)
    return codes, scale


def int8_dequantize(codes, scale, dtype: str) -> np.ndarray:
    """code * scale in fp32, rounded to the pool's ssm dtype, as float64."""
    prod = (np.asarray(codes).astype(np.float32) * np.asarray(scale, np.float32)[..., None, :]).astype(np.float32)
    return round_to(prod.astype(np.float64), dtype)


class Int8StoreRef:
    """Oracle copy of an int8 checkpoint store of `num_entries` entries for a pool's layers:
    codes [E, L, H, P, N] int8, scales [E, L, H, N] fp32, conv [E, L, Cd, W-1] (float64 values
    of the pool's conv dtype)."""

    def __init__(self, pool: PoolRef, num_entries: int):
        L, _, H, P, N = pool.ssm.shape
        self.codes = np.zeros((num_entries, L, H, P, N), np.int8)
        self.scales = np.zeros((num_entries, L, H, N), np.float32)
        self.conv = np.zeros((num_entries, L) + pool.conv.shape[2:])


def int8_store_put(pool: PoolRef, store: Int8StoreRef, layer: int, slots, entries):
    """Quantize slot slots[i] into entry entries[i] (layer < 0: every layer)."""
    layers = range(pool.ssm.shape[0]) if layer < 0 else [layer]
    for l in layers:
        for s, e in zip(slots, entries):
            store.codes[e, l], store.scales[e, l] = int8_quantize(pool.ssm[l, s])
            store.conv[e, l] = pool.conv[l, s]


def int8_store_get(store: Int8StoreRef, pool: PoolRef, layer: int, entries, slots):
    """Dequantize entry entries[i] into slot slots[i] (layer < 0: every layer)."""
    layers = range(pool.ssm.shape[0]) if layer < 0 else [layer]
    for l in layers:
        for e, s in zip(entries, slots):
            pool.ssm[l, s] = int8_dequantize(store.codes[e, l], store.scales[e, l], pool.ssm_dtype)
            pool.conv[l, s] = store.conv[e, l]


# --------------------------------------------------------------------------
# a second recurrent family on the same pool: Mamba1
# --------------------------------------------------------------------------
# [notes] "Mamba" gives the recurrence h_t = exp(Delta_t A) h_{t-1} + Delta_t B_t x_t,
# y_t = C_t h_t; the vLLM state-shape table on the same page gives Mamba1's shapes: a
# conv state (D, W-1) and a recurrent state (D, N).  Read with those shapes, A is a
# (D, N) matrix of negative entries (one decay per channel and state index), Delta a
# per-channel vector (softplus of dt + dt_bias), B_t and C_t length-N vectors shared by
# all channels, and the short conv runs over the D channels of x only (B, C and dt are
# taken as given per token, after whatever produced them).  The D skip term and the
# SiLU(z) gate are as in the Mamba2 path.

class Mamba1PoolRef:
    """Oracle copy of a Mamba1 slot pool: ssm[layer, slot, D, N], conv[layer, slot, D, W-1]."""

    def __init__(self, d_inner: int, d_state: int, conv_kernel: int, num_layers: int, num_slots: int,
                 ssm_dtype: str, conv_dtype: str):
        self.d_inner, self.d_state, self.conv_kernel = d_inner, d_state, conv_kernel
        self.ssm_dtype, self.conv_dtype = ssm_dtype, conv_dtype
        self.ssm = np.zeros((num_layers, num_slots, d_inner, d_state))
        self.conv = np.zeros((num_layers, num_slots, d_inner, conv_kernel - 1))


def mamba1_decode_step(pool: Mamba1PoolRef, layer: int, params: dict, slots, u, z, dt, Bm, Cm, y_dtype: str):
    """One Mamba1 decode token per batch row, in place on the pool.  params: A (D, N) < 0,
    D (D), dt_bias (D), conv_w (D, W), conv_b (D).  Rows: u, z, dt (batch, D); Bm, Cm (batch, N).
    Returns out (batch, D) rounded to y_dtype; slots[b] < 0 is a padding row (zero output)."""
    A, Dk, dt_bias, w, b = (_f64(params[k]) for k in ("A", "D", "dt_bias", "conv_w", "conv_b"))
    out = np.zeros((len(slots), pool.d_inner))
    for r, slot in enumerate(slots):
        if slot < 0:
            continue
        window = np.concatenate([pool.conv[layer, slot], _f64(u[r])[:, None]], axis=1)
        x = silu(b + np.sum(w * window, axis=1))
        delta = softplus(_f64(dt[r]) + dt_bias)
        h = pool.ssm[layer, slot]
        h_new = np.exp(delta[:, None] * A) * h + (delta * x)[:, None] * _f64(Bm[r])[None, :]
        y = h_new @ _f64(Cm[r]) + Dk * x
        out[r] = y * silu(_f64(z[r]))
        pool.ssm[layer, slot] = round_to(h_new, pool.ssm_dtype)
        pool.conv[layer, slot] = round_to(window[:, 1:], pool.conv_dtype)
    return round_to(out, y_dtype)


def mamba1_prefill(pool: Mamba1PoolRef, layer: int, params: dict, cu_seqlens, slots, has_init, start_pos,
                   u, z, dt, Bm, Cm, y_dtype: str, ckpt_interval: int = 0, ckpt_slots=None):
    """Mamba1 prefill of packed sequences: the token-by-token recurrence of mamba1_decode_step with
    the state kept unrounded between tokens; only the final state (slots[s]) and the checkpoint
    states are rounded to the ssm dtype, as in the Mamba2 prefill.  Rows: u, z, dt (T, D); Bm, Cm
    (T, N).  Checkpoint entry k of sequence s takes the state and window after absolute position
    p, the k-th multiple of ckpt_interval with start_pos < p <= start_pos + L."""
    A, Dk, dt_bias, w, b = (_f64(params[k]) for k in ("A", "D", "dt_bias", "conv_w", "conv_b"))
    W = pool.conv_kernel
    out = np.zeros((int(cu_seqlens[-1]), pool.d_inner))
    for s, slot in enumerate(slots):
        t0, t1 = int(cu_seqlens[s]), int(cu_seqlens[s + 1])
        if t1 == t0:
            continue
        sp = int(start_pos[s]) if start_pos is not None else 0
        if has_init[s]:
            h = pool.ssm[layer, slot].copy()
            stream = list(pool.conv[layer, slot].T)         # W-1 rows of D, oldest first
        else:
            h = np.zeros((pool.d_inner, pool.d_state))
            stream = [np.zeros(pool.d_inner) for _ in range(W - 1)]
        for t in range(t0, t1):
            stream.append(_f64(u[t]))
            window = np.stack(stream[-W:], axis=1)
            x = silu(b + np.sum(w * window, axis=1))
            delta = softplus(_f64(dt[t]) + dt_bias)
            h = np.exp(delta[:, None] * A) * h + (delta * x)[:, None] * _f64(Bm[t])[None, :]
            out[t] = (h @ _f64(Cm[t]) + Dk * x) * silu(_f64(z[t]))
            p = sp + (t - t0) + 1
            if ckpt_interval > 0 and ckpt_slots is not None and p % ckpt_interval == 0:
                k = p // ckpt_interval - sp // ckpt_interval - 1
                if 0 <= k < len(ckpt_slots[s]) and ckpt_slots[s][k] >= 0:
                    pool.ssm[layer, ckpt_slots[s][k]] = round_to(h, pool.ssm_dtype)
                    pool.conv[layer, ckpt_slots[s][k]] = round_to(np.stack(stream[-(W - 1):], axis=1),
                                                                  pool.conv_dtype)
        pool.ssm[layer, slot] = round_to(h, pool.ssm_dtype)
        pool.conv[layer, slot] = round_to(np.stack(stream[-(W - 1):], axis=1), pool.conv_dtype)
    return round_to(out, y_dtype)
