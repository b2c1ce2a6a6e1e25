"""GPU parity of the Mamba1 decode step (the pool's second state family) against the oracle."""
import numpy as np
import pytest
import torch

from oracle import mamba2 as orc
from recurrent_state_update_amd import synth
from recurrent_state_update_amd.pool import Pool
from tests.gpu_helpers import TOL, dev, host, log, rel_err, weights

pytestmark = pytest.mark.gpu
TD = {"f32": torch.float32, "bf16": torch.bfloat16}


def _pool(D, N, W, L, S, ssm_dtype, conv_dtype, seed):
    pool = Pool.allocate_mamba1(L, S, D, N, W, TD[ssm_dtype], TD[conv_dtype])
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    for t in (pool.ssm, pool.conv):                  # sentinel bytes everywhere
        b = t.view(torch.uint8)
        b.copy_(torch.randint(0, 256, b.shape, generator=g, device="cuda", dtype=torch.int32).to(torch.uint8))
    return pool


def _raw(t):
    return t.view(torch.uint8).clone()


@pytest.mark.parametrize("D,N,W,ssm_dtype", [(64, 16, 4, "bf16"), (64, 16, 4, "f32"), (48, 8, 2, "f32"),
                                             (32, 64, 3, "bf16"), (16, 256, 4, "f32")])
def test_mamba1_decode_steps_match_the_oracle(D, N, W, ssm_dtype):
    log(f"case: Mamba1 decode D={D} N={N} W={W} ssm={ssm_dtype}, 12 steps")
    rng = np.random.default_rng(800 + N + W)
    params = synth.mamba1_layer_params(rng, D, N, W)
    L, S = 2, 8
    slots = np.array([5, -1, 2, 7], np.int32)
    pool = _pool(D, N, W, L, S, ssm_dtype, "bf16", 81)
    ref = orc.Mamba1PoolRef(D, N, W, L, S, ssm_dtype, "bf16")
    for s in (5, 2, 7):
        h0 = synth.cast_exact(rng.normal(0, 0.1, (D, N)), ssm_dtype)
        w0 = synth.cast_exact(rng.normal(0, 0.1, (D, W - 1)), "bf16")
        pool.ssm[1, s, :, 0] = torch.from_numpy(h0).to(TD[ssm_dtype]).cuda()
        pool.conv[1, s] = torch.from_numpy(w0).to(torch.bfloat16).cuda()
        ref.ssm[1, s], ref.conv[1, s] = h0, w0
    before_s, before_c = _raw(pool.ssm), _raw(pool.conv)
    W_ = weights(params)
    sl = torch.from_numpy(slots).cuda()
    io = ssm_dtype
    y = torch.empty((4, D), dtype=TD[ssm_dtype], device="cuda")
    worst = 0.0
    for t in range(12):
        x, z, dt, Bm, Cm = synth.mamba1_tokens(rng, 4, D, N, io)
        pool.mamba1_decode_step(1, W_, sl, dev(x, io), dev(Bm, io), dev(Cm, io), dev(z, io), dev(dt, io), y,
                                slots_host=slots)
        y_ref = orc.mamba1_decode_step(ref, 1, params, slots, x, z, dt, Bm, Cm, ssm_dtype)
        yh = host(y)
        assert not yh[1].any()                       # padding row
        worst = max(worst, rel_err(yh, y_ref))
    log(f"max rel y error over 12 steps: {worst:.3e}")
    assert worst <= TOL[ssm_dtype]
    for s in (5, 2, 7):
        assert rel_err(host(pool.ssm[1, s, :, 0]), ref.ssm[1, s]) <= TOL[ssm_dtype]
        assert np.array_equal(host(pool.conv[1, s]), ref.conv[1, s])
    # untouched: layer 0 entirely, and the other slots of layer 1
    live = torch.zeros((L, S), dtype=torch.bool, device="cuda")
    live[1, [5, 2, 7]] = True
    for t, b in ((pool.ssm, before_s), (pool.conv, before_c)):
        assert torch.equal(t.view(torch.uint8).view(L, S, -1)[~live], b.view(L, S, -1)[~live])


def test_mamba1_decode_at_the_7b_width_256_of_512_slots():
    """D = 8192, N = 16, W = 4, bf16 pool of 512 slots, 256 rows at permuted slots: sampled rows
    against the oracle, every row's window exact."""
    D, N, W = synth.MAMBA1_D, synth.MAMBA1_N, synth.MAMBA1_W
    log(f"case: Mamba1 decode D={D} N={N}, 256 of 512 slots")
    rng = np.random.default_rng(82)
    params = synth.mamba1_layer_params(rng, D, N, W)
    pool = _pool(D, N, W, 1, 512, "bf16", "bf16", 83)
    slots = rng.permutation(512)[:256].astype(np.int32)
    h0 = synth.cast_exact(rng.normal(0, 0.1, (256, D, N)), "bf16")
    w0 = synth.cast_exact(rng.normal(0, 0.1, (256, D, W - 1)), "bf16")
    pool.ssm[0, torch.from_numpy(slots).long().cuda(), :, 0] = torch.from_numpy(h0).bfloat16().cuda()
    pool.conv[0, torch.from_numpy(slots).long().cuda()] = torch.from_numpy(w0).bfloat16().cuda()
    x, z, dt, Bm, Cm = synth.mamba1_tokens(rng, 256, D, N, "bf16")
    y = torch.empty((256, D), dtype=torch.bfloat16, device="cuda")
    pool.mamba1_decode_step(0, weights(params), torch.from_numpy(slots).cuda(), dev(x, "bf16"), dev(Bm, "bf16"),
                            dev(Cm, "bf16"), dev(z, "bf16"), dev(dt, "bf16"), y, slots_host=slots)
    torch.cuda.synchronize()
    for r in (0, 77, 255):
        ref = orc.Mamba1PoolRef(D, N, W, 1, 1, "bf16", "bf16")
        ref.ssm[0, 0], ref.conv[0, 0] = h0[r], w0[r]
        y_ref = orc.mamba1_decode_step(ref, 0, params, [0], x[r:r + 1], z[r:r + 1], dt[r:r + 1], Bm[r:r + 1],
                                       Cm[r:r + 1], "bf16")
        assert rel_err(host(y[r]), y_ref[0]) <= TOL["bf16"], r
        assert rel_err(host(pool.ssm[0, int(slots[r]), :, 0]), ref.ssm[0, 0]) <= TOL["bf16"], r
    win = host(pool.conv[0, torch.from_numpy(slots).long().cuda()])
    exp = np.concatenate([w0[:, :, 1:], synth.cast_exact(x, "bf16")[:, :, None]], axis=2)
    assert np.array_equal(win, exp)
