"""Shared helpers for the GPU parity tests (pool set-up, sentinels, error metrics)."""
from __future__ import annotations

import numpy as np
import torch

from recurrent_state_update_amd import synth
from recurrent_state_update_amd.pool import LayerWeights, Pool

TORCH_DT = {"f32": torch.float32, "bf16": torch.bfloat16}


def log(msg: str) -> None:
    print(msg, flush=True)


def make_pool(shape: synth.Shape, num_layers: int, num_slots: int, ssm_dtype: str, conv_dtype: str,
              sentinel_seed: int = 1234) -> Pool:
    """A pool whose every byte starts as a seeded random sentinel (NaN payloads included)."""
    g = torch.Generator(device="cuda")
    g.manual_seed(sentinel_seed)
    cd = shape.conv_dim
    ssm = torch.empty((num_layers, num_slots, shape.nheads, shape.head_dim, shape.d_state),
                      dtype=TORCH_DT[ssm_dtype], device="cuda")
    conv = torch.empty((num_layers, num_slots, cd, shape.conv_kernel - 1), dtype=TORCH_DT[conv_dtype],
                       device="cuda")
    for t in (ssm, conv):
        b = t.view(torch.uint8)
        b.copy_(torch.randint(0, 256, b.shape, generator=g, device="cuda", dtype=torch.int32).to(torch.uint8))
    return Pool(ssm, conv, shape.nheads, shape.head_dim, shape.d_state, shape.n_groups, shape.conv_kernel)


def put_slot(pool: Pool, layer: int, slot: int, ssm_vals: np.ndarray, conv_vals: np.ndarray) -> None:
    pool.ssm[layer, slot] = torch.from_numpy(np.asarray(ssm_vals, np.float64)).to(pool.ssm.dtype).cuda()
    pool.conv[layer, slot] = torch.from_numpy(np.asarray(conv_vals, np.float64)).to(pool.conv.dtype).cuda()


def dev(a: np.ndarray, dtype: str) -> torch.Tensor:
    """Exact float64 values -> device tensor of the storage dtype."""
    return synth.to_torch(a, dtype).cuda()


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().to(torch.float64).cpu().numpy()


def rel_err(got, ref) -> float:
    """max |got - ref| / max |ref| over the entries where ref is defined (not NaN)."""
    got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    m = ~np.isnan(ref)
    denom = np.max(np.abs(ref[m])) if m.any() else 1.0
    return float(np.max(np.abs(got[m] - ref[m])) / max(denom, 1e-30)) if m.any() else 0.0


def weights(params: dict) -> LayerWeights:
    return LayerWeights.from_numpy(params)


def raw_bytes(t: torch.Tensor) -> torch.Tensor:
    return t.view(torch.uint8).clone()


def untouched(before: torch.Tensor, after: torch.Tensor, live_slots, layer: int | None = None) -> bool:
    """All slots outside live_slots (in every layer, or one) are byte-identical."""
    L, S = after.shape[0], after.shape[1]
    mask = torch.ones((L, S), dtype=torch.bool, device=after.device)
    for s in live_slots:
        if layer is None:
            mask[:, s] = False
        else:
            mask[layer, s] = False
    b = before.view(L, S, -1)
    a = after.view(torch.uint8).view(L, S, -1)
    return bool(torch.equal(b[mask], a[mask]))


TOL = {"f32": 1e-4, "bf16": 2e-2}
