"""The prefill entry point that allocates nothing (its scratch in the library's static per-GPU
array), through the C ABI, against mamba2_prefill_chunked with a workspace: two calls in a row,
the second smaller, bit for bit."""
import numpy as np
import pytest
import torch

from recurrent_state_update_amd import synth
from tests.gpu_helpers import dev, log, make_pool, put_slot, weights

pytestmark = pytest.mark.gpu


def _case(seed, lens, shape, ssm_dtype, Q, interval):
    rng = np.random.default_rng(seed)
    params = synth.layer_params(rng, shape)
    lens = np.asarray(lens, np.int32)
    n = len(lens)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    start = (np.arange(n, dtype=np.int32) * 37) % interval
    has_init = (np.arange(n) % 2).astype(np.uint8)
    slots = np.arange(n, dtype=np.int32) * 3
    counts = (start + lens) // interval - start // interval
    ck = np.full((n, max(1, int(counts.max()))), -1, np.int32)
    free = iter([s for s in range(3 * n, 3 * n + 64)])
    for i in range(n):
        for k in range(counts[i]):
            ck[i, k] = next(free)
    u, z, dt = synth._tokens(rng, shape, int(cu[-1]), ssm_dtype)
    ssm0 = synth.cast_exact(rng.normal(0, 0.1, (n, shape.nheads, shape.head_dim, shape.d_state)), ssm_dtype)
    conv0 = synth.cast_exact(rng.normal(0, 0.1, (n, shape.conv_dim, shape.conv_kernel - 1)), "bf16")
    return dict(params=params, cu=cu, start=start, has_init=has_init, slots=slots, ck=ck, u=u, z=z, dt=dt,
                ssm0=ssm0, conv0=conv0, Q=Q, interval=interval)


def _run(pool_fn, c, shape, ssm_dtype, noalloc):
    pool = pool_fn()
    for i, s in enumerate(c["slots"]):
        put_slot(pool, 0, int(s), c["ssm0"][i], c["conv0"][i])
    T = int(c["cu"][-1])
    y = torch.full((T, shape.intermediate), float("nan"), dtype=synth._TORCH[ssm_dtype], device="cuda")
    x, B, C = pool.split_xbc(dev(c["u"], ssm_dtype))
    args = (0, weights(c["params"]), c["cu"], c["slots"], c["has_init"], x, B, C, dev(c["z"], ssm_dtype),
            dev(c["dt"], ssm_dtype), y)
    kw = dict(start_pos=c["start"], chunk_size=c["Q"], ckpt_interval=c["interval"], ckpt_slots=c["ck"])
    if noalloc:
        pool.prefill_noalloc(*args, **kw)
    else:
        pool.prefill(*args, **kw)
    torch.cuda.synchronize()
    return pool, y


@pytest.mark.parametrize("ssm_dtype", ["bf16", "f32"])
def test_noalloc_prefill_equals_the_workspace_prefill_twice(ssm_dtype):
    shape = synth.Shape(16, 64, 128, 4, 4)
    big = _case(601, [700, 1, 255, 513, 96], shape, ssm_dtype, 128, 200)
    small = _case(602, [33, 130], shape, ssm_dtype, 64, 50)
    for name, c in (("larger", big), ("smaller", small)):
        log(f"case: no-alloc prefill, {name} input, ssm={ssm_dtype}, {int(c['cu'][-1])} tokens")
        mk = lambda: make_pool(shape, 1, 80, ssm_dtype, "bf16", sentinel_seed=5)
        pa, ya = _run(mk, c, shape, ssm_dtype, noalloc=False)
        pb, yb = _run(mk, c, shape, ssm_dtype, noalloc=True)
        bits = torch.int16 if ssm_dtype == "bf16" else torch.int32
        assert torch.equal(ya.view(bits), yb.view(bits))
        assert torch.equal(pa.ssm.view(torch.uint8), pb.ssm.view(torch.uint8))
        assert torch.equal(pa.conv.view(torch.uint8), pb.conv.view(torch.uint8))


def test_noalloc_prefill_refuses_a_call_beyond_its_scratch():
    shape = synth.NEMOTRON_H
    pool = make_pool(shape, 1, 4, "bf16", "bf16")
    T = 16384
    cu = np.array([0, T], np.int32)
    need = pool.workspace_size(cu, 256)
    assert need > 64 * 1024 * 1024
    x = torch.zeros((T, shape.conv_dim), dtype=torch.bfloat16, device="cuda")
    xx, B, C = pool.split_xbc(x)
    z = torch.zeros((T, shape.intermediate), dtype=torch.bfloat16, device="cuda")
    dt = torch.zeros((T, shape.nheads), dtype=torch.bfloat16, device="cuda")
    y = torch.zeros((T, shape.intermediate), dtype=torch.bfloat16, device="cuda")
    before = pool.ssm.view(torch.uint8).clone()
    with pytest.raises(Exception, match="static scratch"):
        pool.prefill_noalloc(0, weights(synth.layer_params(np.random.default_rng(0), shape)), cu, [1], [0], xx, B, C,
                             z, dt, y, chunk_size=256)
    torch.cuda.synchronize()
    assert torch.equal(before, pool.ssm.view(torch.uint8))
