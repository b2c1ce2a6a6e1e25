"""Seeded synthetic inputs for the Mamba2 slot-pool workloads.

This module only draws random numbers and lays them out.  It holds none of
the method's arithmetic, so both sides of a parity check (the CPU oracle and
the HIP path) may take their inputs from it.  Normal values are drawn as
float32 with ``numpy.random.default_rng(...).standard_normal(dtype=float32)``,
uniform values as float64; both are then cast to their storage dtype with
torch's CPU casts (-> float32 -> bfloat16, round-to-nearest-even at each step).
Large arrays (states, tokens) are float32 holding values exactly representable
in the dtype named beside them (bf16 values are exact in float32); layer
parameters are float64 arrays of fp32-exact values.

Shapes follow the Nemotron-H Mamba2 layer the first page prints in its model
config (128 heads of 64 channels, state size 128, 8 groups, conv width 4,
d_inner 8192), and a tiny layer of the same structure.

Distributions (one rule for every workload):
  pre-conv inputs u = [x | B | C], gate z, and dt    ~ N(0, 1)
  dt_bias ~ U(-4, -2);  A = -exp(U(0, ln 16));  D ~ N(0, 1)
  conv weight and bias ~ U(-0.5, 0.5)   (PyTorch Conv1d's default bound 1/sqrt(W))
  live initial SSM state and conv window ~ N(0, 0.1)
  slots that a call must not touch hold random bytes (sentinels, NaNs included)
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np
import torch

DTYPES = ("f32", "bf16")
_TORCH = {"f32": torch.float32, "bf16": torch.bfloat16}
_NBYTES = {"f32": 4, "bf16": 2}


@dataclass(frozen=True)
class Shape:
    """Mamba2 layer shape: H heads of P channels, state N, G groups, conv W."""

    nheads: int
    head_dim: int
    d_state: int
    n_groups: int
    conv_kernel: int

    @property
    def intermediate(self) -> int:
        return self.nheads * self.head_dim

    @property
    def conv_dim(self) -> int:
        return self.intermediate + 2 * self.n_groups * self.d_state


TINY = Shape(nheads=8, head_dim=16, d_state=16, n_groups=1, conv_kernel=4)
NEMOTRON_H = Shape(nheads=128, head_dim=64, d_state=128, n_groups=8, conv_kernel=4)


def cast_exact(a, dtype: str) -> np.ndarray:
    """Round values to ``dtype`` (torch CPU casts) and return them as a float32 array."""
    a = np.asarray(a)
    if a.dtype != np.float32:
        a = a.astype(np.float64)
    t = torch.from_numpy(np.ascontiguousarray(a)).to(torch.float32)
    if dtype == "bf16":
        t = t.to(torch.bfloat16).to(torch.float32)
    elif dtype != "f32":
        raise ValueError(dtype)
    return t.numpy()


def normal(rng: np.random.Generator, shape, std: float = 1.0) -> np.ndarray:
    """float32 N(0, std^2) draws."""
    a = rng.standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return a


def to_torch(a: np.ndarray, dtype: str) -> torch.Tensor:
    """Values exact in ``dtype`` -> CPU tensor of the storage dtype."""
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(_TORCH[dtype])


def layer_params(rng: np.random.Generator, shape: Shape) -> dict:
    """Per-layer parameters drawn in a fixed order; float64 arrays of fp32-exact values."""
    H, Cd, W = shape.nheads, shape.conv_dim, shape.conv_kernel
    dt_bias = rng.uniform(-4.0, -2.0, H)
    A = -np.exp(rng.uniform(0.0, math.log(16.0), H))
    D = rng.standard_normal(H)   # float64: parameters are small
    conv_w = rng.uniform(-0.5, 0.5, (Cd, W))
    conv_b = rng.uniform(-0.5, 0.5, Cd)
    return {k: cast_exact(v, "f32").astype(np.float64) for k, v in
            dict(A=A, D=D, dt_bias=dt_bias, conv_w=conv_w, conv_b=conv_b).items()}


# A Mamba1 layer for the second state family of the pool: D channels, state size N, conv W
# (d_inner 8192, d_state 16, conv 4: the width of the 7B-class Mamba1 models).
MAMBA1_D, MAMBA1_N, MAMBA1_W = 8192, 16, 4


def mamba1_layer_params(rng: np.random.Generator, D: int, N: int, W: int) -> dict:
    """Mamba1 parameters drawn in a fixed order, fp32-exact float64: A (D, N) < 0, D, dt_bias,
    conv_b (D), conv_w (D, W); same value ranges as the Mamba2 layer."""
    dt_bias = rng.uniform(-4.0, -2.0, D)
    A = -np.exp(rng.uniform(0.0, math.log(16.0), (D, N)))
    Dk = rng.standard_normal(D)
    conv_w = rng.uniform(-0.5, 0.5, (D, W))
    conv_b = rng.uniform(-0.5, 0.5, D)
    return {k: cast_exact(v, "f32").astype(np.float64) for k, v in
            dict(A=A, D=Dk, dt_bias=dt_bias, conv_w=conv_w, conv_b=conv_b).items()}


def mamba1_tokens(rng: np.random.Generator, n: int, D: int, N: int, io_dtype: str):
    """n Mamba1 token rows: raw x (D), z (D), dt (D), B (N), C (N), N(0, 1), io-dtype exact."""
    return tuple(cast_exact(rng.standard_normal(s), io_dtype) for s in ((n, D), (n, D), (n, D), (n, N), (n, N)))


def sentinel_bytes(rng: np.random.Generator, nbytes: int) -> np.ndarray:
    return rng.integers(0, 256, nbytes, dtype=np.uint8)


def pool_bytes(shape: Shape, num_layers: int, num_slots: int, ssm_dtype: str, conv_dtype: str):
    ssm = num_layers * num_slots * shape.nheads * shape.head_dim * shape.d_state * _NBYTES[ssm_dtype]
    conv = num_layers * num_slots * shape.conv_dim * (shape.conv_kernel - 1) * _NBYTES[conv_dtype]
    return ssm, conv


def _live_state(rng, shape: Shape, n: int, ssm_dtype: str, conv_dtype: str):
    H, P, N, Cd, W = shape.nheads, shape.head_dim, shape.d_state, shape.conv_dim, shape.conv_kernel
    ssm = cast_exact(normal(rng, (n, H, P, N), 0.1), ssm_dtype)
    conv = cast_exact(normal(rng, (n, Cd, W - 1), 0.1), conv_dtype)
    return ssm, conv


def _tokens(rng, shape: Shape, T: int, io_dtype: str):
    u = cast_exact(normal(rng, (T, shape.conv_dim)), io_dtype)
    z = cast_exact(normal(rng, (T, shape.intermediate)), io_dtype)
    dt = cast_exact(normal(rng, (T, shape.nheads)), io_dtype)
    return u, z, dt


def tiny_workload(seed: int = 0) -> dict:
    """Tiny fp32 layer: 4 sequences in an 8-slot pool at slots [5, 0, 3, 7].

    64 decode steps per sequence; the same 64 tokens per sequence also form a
    packed prefill (cu_seqlens [0, 64, 128, 192, 256]) with chunk 16.
    """
    shape = TINY
    rng = np.random.default_rng(seed)
    params = layer_params(rng, shape)
    slots = np.array([5, 0, 3, 7], dtype=np.int32)
    ssm0, conv0 = _live_state(rng, shape, len(slots), "f32", "f32")
    steps, batch = 64, len(slots)
    u = cast_exact(normal(rng, (steps, batch, shape.conv_dim)), "f32")
    z = cast_exact(normal(rng, (steps, batch, shape.intermediate)), "f32")
    dt = cast_exact(normal(rng, (steps, batch, shape.nheads)), "f32")
    ssm_bytes, conv_bytes = pool_bytes(shape, 1, 8, "f32", "f32")
    return dict(
        name="tiny fp32 layer (H=8, P=16, N=16, G=1, W=4), 4 of 8 slots, 64 steps",
        shape=shape, num_layers=1, num_slots=8, ssm_dtype="f32", conv_dtype="f32",
        io_dtype="f32", y_dtype="f32", params=params, slots=slots,
        ssm0=ssm0, conv0=conv0, u=u, z=z, dt=dt, chunk=16,
        cu_seqlens=np.arange(0, steps * batch + 1, steps, dtype=np.int32),
        sentinel_ssm=sentinel_bytes(rng, ssm_bytes), sentinel_conv=sentinel_bytes(rng, conv_bytes),
    )


def decode_workload(seed: int = 1, batch: int = 256, num_slots: int = 512,
                    shape: Shape = NEMOTRON_H, ssm_dtype: str = "bf16", conv_dtype: str = "bf16",
                    io_dtype: str = "bf16", with_state: bool = True) -> dict:
    """One decode token for ``batch`` sequences at randomly permuted slots of a pool."""
    rng = np.random.default_rng(seed)
    params = layer_params(rng, shape)
    slots = rng.permutation(num_slots)[:batch].astype(np.int32)
    out = dict(name=f"decode, {batch} sequences in a {num_slots}-slot pool",
               shape=shape, num_layers=1, num_slots=num_slots, ssm_dtype=ssm_dtype,
               conv_dtype=conv_dtype, io_dtype=io_dtype, y_dtype=io_dtype, params=params, slots=slots)
    if with_state:
        out["ssm0"], out["conv0"] = _live_state(rng, shape, batch, ssm_dtype, conv_dtype)
    else:
        out["state_seed"] = int(rng.integers(0, 2**31))
    out["u"], out["z"], out["dt"] = _tokens(rng, shape, batch, io_dtype)
    return out


def prefill_workload(seed: int = 2, L: int = 8192, chunk: int = 256, slot: int = 17,
                     num_slots: int = 512, shape: Shape = NEMOTRON_H) -> dict:
    """One sequence prefilled from a zero state; final state goes to ``slot`` (pre-filled with NaN)."""
    rng = np.random.default_rng(seed)
    params = layer_params(rng, shape)
    u, z, dt = _tokens(rng, shape, L, "bf16")
    return dict(name=f"prefill, one sequence of {L} tokens, chunk {chunk}", shape=shape,
                num_layers=1, num_slots=num_slots, ssm_dtype="bf16", conv_dtype="bf16",
                io_dtype="bf16", y_dtype="bf16", params=params,
                slots=np.array([slot], np.int32), cu_seqlens=np.array([0, L], np.int32),
                has_init=np.zeros(1, np.uint8), start_pos=np.zeros(1, np.int32),
                u=u, z=z, dt=dt, chunk=chunk)


def mixed_layout(seed: int = 3, n_prefill: int = 32, n_decode: int = 224, num_slots: int = 512,
                 interval: int = 1024, shape: Shape = NEMOTRON_H, lmin: int = 128, lmax: int = 4096):
    """The mixed batch without its token data: (rng, params, prefill lengths, prefill slots,
    decode slots, checkpoint slots); the rng is left where the token draws begin."""
    rng = np.random.default_rng(seed)
    params = layer_params(rng, shape)
    lens = rng.integers(lmin, lmax + 1, n_prefill).astype(np.int32)
    perm = rng.permutation(num_slots).astype(np.int32)
    p_slots, d_slots = perm[:n_prefill], perm[n_prefill:n_prefill + n_decode]
    free = np.sort(perm[n_prefill + n_decode:])
    n_ck = lens // interval
    max_ck = max(1, int(n_ck.max()))
    ck = np.full((n_prefill, max_ck), -1, np.int32)
    it = iter(free.tolist())
    for i in range(n_prefill):
        for k in range(n_ck[i]):
            ck[i, k] = next(it)
    return rng, params, lens, p_slots, d_slots, ck


def mixed_workload(seed: int = 3, n_prefill: int = 32, n_decode: int = 224, num_slots: int = 512,
                   interval: int = 1024, chunk: int = 256, shape: Shape = NEMOTRON_H,
                   lmin: int = 128, lmax: int = 4096) -> dict:
    """Continuous batch: varlen-packed prefills from zero state plus single-token decodes.

    Checkpoint slots are taken from the free slots in ascending order, in
    (sequence, checkpoint) order; a prefill of L tokens checkpoints at every
    multiple of ``interval`` in (0, L].
    """
    rng, params, lens, p_slots, d_slots, ck = mixed_layout(seed, n_prefill, n_decode, num_slots, interval, shape,
                                                           lmin, lmax)
    T = int(lens.sum())
    u, z, dt = _tokens(rng, shape, T, "bf16")
    d_ssm0, d_conv0 = _live_state(rng, shape, n_decode, "bf16", "bf16")
    du, dz, ddt = _tokens(rng, shape, n_decode, "bf16")
    return dict(name=f"mixed batch: {n_prefill} prefills (U({lmin},{lmax})) + {n_decode} decodes",
                shape=shape, num_layers=1, num_slots=num_slots, ssm_dtype="bf16", conv_dtype="bf16",
                io_dtype="bf16", y_dtype="bf16", params=params, chunk=chunk, interval=interval,
                lens=lens, cu_seqlens=np.concatenate([[0], np.cumsum(lens)]).astype(np.int32),
                prefill_slots=p_slots, decode_slots=d_slots, ckpt_slots=ck,
                has_init=np.zeros(n_prefill, np.uint8), start_pos=np.zeros(n_prefill, np.int32),
                u=u, z=z, dt=dt, decode_ssm0=d_ssm0, decode_conv0=d_conv0,
                decode_u=du, decode_z=dz, decode_dt=ddt)


LONG_BLOCK = 4096


def long_layer_params(layer: int, seed: int = 4, shape: Shape = NEMOTRON_H) -> dict:
    """Independent seeded parameters of layer ``layer`` of the 48-layer long-context stack."""
    return layer_params(np.random.default_rng([seed, 1 + layer]), shape)


def long_token_block(blk: int, seed: int = 4, shape: Shape = NEMOTRON_H):
    """Tokens [blk*4096, (blk+1)*4096) of the packed long-context input (bf16 u, z, dt)."""
    return _tokens(np.random.default_rng([seed, 0, blk]), shape, LONG_BLOCK, "bf16")


def long_workload(seqs: int = 2, L: int = 131072, layers: int = 48, chunk: int = 256) -> dict:
    """2 x 131072 tokens through 48 independently parameterised layers, fp32 SSM state."""
    assert L % LONG_BLOCK == 0
    return dict(name=f"long context: {seqs} x {L} tokens, {layers} layers, fp32 state",
                shape=NEMOTRON_H, num_layers=layers, num_slots=seqs, ssm_dtype="f32",
                conv_dtype="bf16", io_dtype="bf16", y_dtype="f32", chunk=chunk, L=L, seqs=seqs,
                cu_seqlens=np.arange(0, seqs * L + 1, L, dtype=np.int32),
                slots=np.arange(seqs, dtype=np.int32), has_init=np.zeros(seqs, np.uint8),
                start_pos=np.zeros(seqs, np.int32), blocks=seqs * L // LONG_BLOCK)


def random_problem(rng: np.random.Generator, shape: Shape, T: int, io_dtype: str = "f32",
                   state_std: float = 0.1):
    """Small random problem used by property tests: params, one initial state and T tokens."""
    params = layer_params(rng, shape)
    ssm0 = normal(rng, (shape.nheads, shape.head_dim, shape.d_state), state_std)
    conv0 = normal(rng, (shape.conv_dim, shape.conv_kernel - 1), state_std)
    u, z, dt = _tokens(rng, shape, T, io_dtype)
    f64 = lambda a: np.asarray(a, np.float64)
    return params, f64(cast_exact(ssm0, "f32")), f64(cast_exact(conv0, "f32")), f64(u), f64(z), f64(dt)
