"""GPU checks of the multi-token (speculative) decode: equal, bit for bit, to the same tokens run
as single decode steps on the GPU; within tolerance of the oracle with exact windows and
placement; padding rows and dropped snapshots."""
import numpy as np
import pytest
import torch

from oracle import mamba2 as orc
from recurrent_state_update_amd import synth
from tests.gpu_helpers import TOL, dev, host, log, make_pool, put_slot, raw_bytes, rel_err, untouched, weights

pytestmark = pytest.mark.gpu


def _i32(v):
    return torch.tensor(np.asarray(v, np.int32), device="cuda")


def _single_steps(pool, W, slot_in, K, rows_u, rows_z, rows_dt, io, y_dtype, work):
    """Run K single decode steps on a copy of slot_in kept in slot `work`; returns y rows and the
    snapshots (ssm, conv) after each token."""
    pool.ssm[0, work] = pool.ssm[0, slot_in]
    pool.conv[0, work] = pool.conv[0, slot_in]
    ys, snaps = [], []
    sl = _i32([work])
    for t in range(K):
        x, B, C = pool.split_xbc(rows_u[t:t + 1])
        y = torch.empty((1, pool.intermediate), dtype=y_dtype, device="cuda")
        pool.decode_step(0, W, sl, x, B, C, rows_z[t:t + 1], rows_dt[t:t + 1], y)
        ys.append(y)
        snaps.append((pool.ssm[0, work].clone(), pool.conv[0, work].clone()))
    return torch.cat(ys), snaps


@pytest.mark.parametrize("ssm_dtype,K", [("bf16", 4), ("f32", 3), ("bf16", 8)])
def test_multi_token_decode_equals_single_steps_bit_for_bit(ssm_dtype, K):
    sh = synth.Shape(16, 64, 128, 2, 4)
    log(f"case: multi-token decode vs single steps ssm={ssm_dtype} K={K}")
    rng = np.random.default_rng(700 + K)
    params = synth.layer_params(rng, sh)
    batch = 5
    pool = make_pool(sh, 1, 96, ssm_dtype, "bf16", sentinel_seed=71)
    ins = [3, 10, 17, 24, 31]
    for s in ins:
        put_slot(pool, 0, s, synth.cast_exact(rng.normal(0, 0.1, (sh.nheads, sh.head_dim, sh.d_state)), ssm_dtype),
                 synth.cast_exact(rng.normal(0, 0.1, (sh.conv_dim, sh.conv_kernel - 1)), "bf16"))
    outs = np.array([[40 + 8 * b + t for t in range(K)] for b in range(batch)], np.int32)
    u, z, dt = synth._tokens(rng, sh, batch * K, ssm_dtype)
    W = weights(params)
    ud, zd, dd = dev(u, ssm_dtype), dev(z, ssm_dtype), dev(dt, ssm_dtype)
    ydt = torch.float32 if ssm_dtype == "f32" else torch.bfloat16
    # single steps first, on a copy of each input slot (slot 95 as the working slot)
    refs = [_single_steps(pool, W, ins[b], K, ud[b * K:(b + 1) * K], zd[b * K:(b + 1) * K], dd[b * K:(b + 1) * K],
                          ssm_dtype, ydt, 95) for b in range(batch)]
    x, B, C = pool.split_xbc(ud)
    y = torch.empty((batch * K, sh.intermediate), dtype=ydt, device="cuda")
    before = raw_bytes(pool.ssm)
    pool.decode_multi(0, W, _i32(ins), _i32(outs), x, B, C, zd, dd, y, slots_in_host=ins, slots_out_host=outs)
    torch.cuda.synchronize()
    bits = torch.int16 if ssm_dtype == "bf16" else torch.int32
    for b in range(batch):
        y_ref, snaps = refs[b]
        assert torch.equal(y[b * K:(b + 1) * K].view(bits), y_ref.view(bits)), b
        for t in range(K):
            assert torch.equal(pool.ssm[0, outs[b, t]].view(bits), snaps[t][0].view(bits)), (b, t)
            assert torch.equal(pool.conv[0, outs[b, t]], snaps[t][1]), (b, t)
    assert untouched(before, pool.ssm, outs.ravel().tolist())        # input slots too


def test_multi_token_decode_matches_the_oracle_with_padding_and_dropped_snapshots():
    sh = synth.Shape(6, 32, 64, 3, 3)
    K = 4
    log("case: multi-token decode vs oracle, padding row, dropped snapshots")
    rng = np.random.default_rng(72)
    params = synth.layer_params(rng, sh)
    pool = make_pool(sh, 1, 24, "f32", "f32", sentinel_seed=73)
    ref = orc.PoolRef(sh, 1, 24, "f32", "f32")
    ins = np.array([2, -1, 5], np.int32)
    outs = np.array([[8, 9, 10, 2], [11, 12, 13, 14], [-1, 15, -1, 16]], np.int32)   # row 0 ends in place
    for s in (2, 5):
        st = synth.cast_exact(rng.normal(0, 0.1, (sh.nheads, sh.head_dim, sh.d_state)), "f32")
        cv = synth.cast_exact(rng.normal(0, 0.1, (sh.conv_dim, sh.conv_kernel - 1)), "f32")
        put_slot(pool, 0, s, st, cv)
        ref.ssm[0, s], ref.conv[0, s] = st, cv
    u, z, dt = synth._tokens(rng, sh, 3 * K, "f32")
    before_s, before_c = raw_bytes(pool.ssm), raw_bytes(pool.conv)
    x, B, C = pool.split_xbc(dev(u, "f32"))
    y = torch.full((3 * K, sh.intermediate), float("nan"), dtype=torch.float32, device="cuda")
    pool.decode_multi(0, weights(params), _i32(ins), _i32(outs), x, B, C, dev(z, "f32"), dev(dt, "f32"), y,
                      slots_in_host=ins, slots_out_host=outs)
    torch.cuda.synchronize()
    sh3 = lambda a: a.reshape(3, K, -1)
    y_ref = orc.decode_multi(ref, 0, params, ins, outs, sh3(u), sh3(z), sh3(dt), "f32")
    yh = host(y).reshape(3, K, -1)
    assert rel_err(yh, y_ref) <= TOL["f32"]
    assert not yh[1].any()                                            # padding row
    written = [8, 9, 10, 2, 15, 16]
    for s in written:
        assert rel_err(host(pool.ssm[0, s]), ref.ssm[0, s]) <= TOL["f32"], s
        assert np.array_equal(host(pool.conv[0, s]), ref.conv[0, s]), s
    assert untouched(before_s, pool.ssm, written) and untouched(before_c, pool.conv, written)


def test_multi_token_decode_rejects_aliasing_host_slots():
    sh = synth.TINY
    pool = make_pool(sh, 1, 8, "f32", "f32")
    W = weights(synth.layer_params(np.random.default_rng(74), sh))
    u = torch.zeros((4, sh.conv_dim), device="cuda")
    x, B, C = pool.split_xbc(u)
    zz = torch.zeros((4, sh.intermediate), device="cuda")
    dd = torch.zeros((4, sh.nheads), device="cuda")
    y = torch.empty((4, sh.intermediate), device="cuda")
    from recurrent_state_update_amd.pool import Mamba2Error
    for ins, outs in (([0, 1], [[2, 3], [4, 0]]),       # an output is another row's input
                      ([0, 1], [[2, 3], [3, 4]]),       # an output twice
                      ([0, 0], [[2, 3], [4, 5]])):      # an input twice
        with pytest.raises(Mamba2Error):
            pool.decode_multi(0, W, _i32(ins), _i32(outs), x, B, C, zz, dd, y, slots_in_host=ins,
                              slots_out_host=outs)


@pytest.mark.parametrize("K,n", [(4, 256), (8, 64)])
def test_layer_shape_equals_single_steps(K, n):
    """The Nemotron-H layer shape: 256 sequences of a 1280-slot bf16 pool with 4 tokens each (a
    verified token and 3 drafts; the benchmark's size), and 64 sequences with 8 tokens (75 KB of
    LDS per workgroup, above the default 64 KiB), against K single-step launches over all rows."""
    w = synth.decode_workload(1)
    sh = w["shape"]
    log(f"case: multi-token decode, {n} sequences x {K} tokens, Nemotron-H layer shape")
    g = torch.Generator(device="cuda")
    g.manual_seed(75)
    pool = make_pool(sh, 1, 1280, "bf16", "bf16", sentinel_seed=76)
    perm = torch.randperm(1280, generator=g, device="cuda").to(torch.int32)
    ins, outs = perm[:n], perm[n:n + n * K].reshape(n, K)
    pool.ssm[0, ins.long()] = (torch.randn((n,) + tuple(pool.ssm.shape[2:]), generator=g, device="cuda") * 0.1).bfloat16()
    pool.conv[0, ins.long()] = (torch.randn((n,) + tuple(pool.conv.shape[2:]), generator=g, device="cuda") * 0.1).bfloat16()
    u = torch.randn((n * K, sh.conv_dim), generator=g, device="cuda").bfloat16()
    z = torch.randn((n * K, sh.intermediate), generator=g, device="cuda").bfloat16()
    dt = torch.randn((n * K, sh.nheads), generator=g, device="cuda").bfloat16()
    W = weights(w["params"])
    # single steps on a second pool holding the same input states
    ref = make_pool(sh, 1, 1280, "bf16", "bf16", sentinel_seed=76)
    ref.ssm.copy_(pool.ssm)
    ref.conv.copy_(pool.conv)
    y_ref = torch.empty((n, K, sh.intermediate), dtype=torch.bfloat16, device="cuda")
    ref_snap = []
    for t in range(K):
        rows = torch.arange(n, device="cuda") * K + t
        x, B, C = ref.split_xbc(u[rows].contiguous())
        yt = torch.empty((n, sh.intermediate), dtype=torch.bfloat16, device="cuda")
        ref.decode_step(0, W, ins, x, B, C, z[rows].contiguous(), dt[rows].contiguous(), yt)
        y_ref[:, t] = yt
        ref_snap.append((ref.ssm[0, ins.long()].clone(), ref.conv[0, ins.long()].clone()))
    x, B, C = pool.split_xbc(u)
    y = torch.empty((n * K, sh.intermediate), dtype=torch.bfloat16, device="cuda")
    pool.decode_multi(0, W, ins, outs.contiguous(), x, B, C, z, dt, y)
    torch.cuda.synchronize()
    assert torch.equal(y.view(n, K, -1).view(torch.int16), y_ref.view(torch.int16))
    for t in range(K):
        assert torch.equal(pool.ssm[0, outs[:, t].long()].view(torch.int16), ref_snap[t][0].view(torch.int16)), t
        assert torch.equal(pool.conv[0, outs[:, t].long()], ref_snap[t][1]), t
