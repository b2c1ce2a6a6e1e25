"""GPU parity of the fused decode step against the CPU oracle (through the C ABI)."""
import numpy as np
import pytest
import torch

from oracle import mamba2 as orc
from recurrent_state_update_amd import synth
from tests.gpu_helpers import (TOL, dev, host, log, make_pool, put_slot, raw_bytes, rel_err, untouched,
                               weights)

pytestmark = pytest.mark.gpu


def test_tiny_fp32_64_decode_steps():
    w = synth.tiny_workload(0)
    sh, slots = w["shape"], w["slots"]
    log(f"case: {w['name']}")
    pool = make_pool(sh, 1, 8, "f32", "f32")
    for i, s in enumerate(slots):
        put_slot(pool, 0, int(s), w["ssm0"][i], w["conv0"][i])
    ref = orc.PoolRef(sh, 1, 8, "f32", "f32")
    ref.ssm[0, slots], ref.conv[0, slots] = w["ssm0"], w["conv0"]
    before_s, before_c = raw_bytes(pool.ssm), raw_bytes(pool.conv)
    W = weights(w["params"])
    sl = torch.from_numpy(slots).cuda()
    y = torch.empty((4, sh.intermediate), dtype=torch.float32, device="cuda")
    worst = 0.0
    for t in range(64):
        u = dev(w["u"][t], "f32")
        x, B, C = pool.split_xbc(u)
        pool.decode_step(0, W, sl, x, B, C, dev(w["z"][t], "f32"), dev(w["dt"][t], "f32"), y, slots_host=slots)
        y_ref = orc.decode_step(ref, 0, w["params"], slots, w["u"][t], w["z"][t], w["dt"][t], "f32")
        worst = max(worst, rel_err(host(y), y_ref))
    log(f"max rel y error over 64 steps: {worst:.3e}")
    assert worst <= TOL["f32"]
    for i, s in enumerate(slots):
        assert rel_err(host(pool.ssm[0, s]), ref.ssm[0, s]) <= TOL["f32"]
        assert np.array_equal(host(pool.conv[0, s]), ref.conv[0, s])      # window = exact copies
    assert untouched(before_s, pool.ssm, slots) and untouched(before_c, pool.conv, slots)


@pytest.fixture(scope="module")
def decode_8b():
    w = synth.decode_workload(1)
    return w


def test_8b_shape_decode_256_of_512_slots(decode_8b):
    w = decode_8b
    sh, slots = w["shape"], w["slots"]
    log(f"case: {w['name']} (H=128, P=64, N=128, G=8, bf16 state)")
    pool = make_pool(sh, 1, 512, "bf16", "bf16")
    for i, s in enumerate(slots):
        put_slot(pool, 0, int(s), w["ssm0"][i], w["conv0"][i])
    before_s, before_c = raw_bytes(pool.ssm), raw_bytes(pool.conv)
    u = dev(w["u"], "bf16")
    x, B, C = pool.split_xbc(u)
    y = torch.empty((256, sh.intermediate), dtype=torch.bfloat16, device="cuda")
    pool.decode_step(0, weights(w["params"]), torch.from_numpy(slots).cuda(), x, B, C,
                     dev(w["z"], "bf16"), dev(w["dt"], "bf16"), y, slots_host=slots)
    torch.cuda.synchronize()
    ref = orc.PoolRef(sh, 1, 256, "bf16", "bf16")
    ref.ssm[0], ref.conv[0] = w["ssm0"], w["conv0"]
    y_ref = orc.decode_step(ref, 0, w["params"], np.arange(256), w["u"], w["z"], w["dt"], "bf16")
    e = rel_err(host(y), y_ref)
    log(f"y rel error {e:.3e}")
    assert e <= TOL["bf16"]
    es = max(rel_err(host(pool.ssm[0, int(s)]), ref.ssm[0, i]) for i, s in enumerate(slots))
    log(f"max state rel error {es:.3e}")
    assert es <= TOL["bf16"]
    for i, s in enumerate(slots):
        assert np.array_equal(host(pool.conv[0, int(s)]), ref.conv[0, i])
    assert untouched(before_s, pool.ssm, slots) and untouched(before_c, pool.conv, slots)


def test_padding_rows_and_out_of_range_slots_are_no_ops():
    sh = synth.Shape(16, 64, 128, 2, 4)
    rng = np.random.default_rng(5)
    params = synth.layer_params(rng, sh)
    pool = make_pool(sh, 2, 6, "bf16", "bf16")
    ssm0 = synth.cast_exact(rng.normal(0, 0.1, (sh.nheads, sh.head_dim, sh.d_state)), "bf16")
    conv0 = synth.cast_exact(rng.normal(0, 0.1, (sh.conv_dim, 3)), "bf16")
    put_slot(pool, 1, 4, ssm0, conv0)
    before_s, before_c = raw_bytes(pool.ssm), raw_bytes(pool.conv)
    slots = np.array([-1, 4, 99, -7], np.int32)          # device-side: out of range = padding
    u = synth.cast_exact(rng.standard_normal((4, sh.conv_dim)), "bf16")
    z = synth.cast_exact(rng.standard_normal((4, sh.intermediate)), "bf16")
    dt = synth.cast_exact(rng.standard_normal((4, sh.nheads)), "bf16")
    y = torch.full((4, sh.intermediate), 7.0, dtype=torch.float32, device="cuda")
    x, B, C = pool.split_xbc(dev(u, "bf16"))
    pool.decode_step(1, weights(params), torch.from_numpy(slots).cuda(), x, B, C, dev(z, "bf16"),
                     dev(dt, "bf16"), y)
    yh = host(y)
    assert np.all(yh[[0, 2, 3]] == 0)
    ref = orc.PoolRef(sh, 1, 1, "bf16", "bf16")
    ref.ssm[0, 0], ref.conv[0, 0] = ssm0, conv0
    y_ref = orc.decode_step(ref, 0, params, [0], u[1:2], z[1:2], dt[1:2], "f32")
    assert rel_err(yh[1], y_ref[0]) <= TOL["bf16"]
    assert untouched(before_s, pool.ssm, [4], layer=1) and untouched(before_c, pool.conv, [4], layer=1)


def test_decode_is_deterministic_and_batch_invariant(decode_8b):
    """Same inputs give the same bits, and a row's result does not depend on the rest of the batch."""
    w = decode_8b
    sh, slots = w["shape"], w["slots"][:64]
    u, z, dt = dev(w["u"][:64], "bf16"), dev(w["z"][:64], "bf16"), dev(w["dt"][:64], "bf16")
    W = weights(w["params"])
    outs = []
    for order in (np.arange(64), np.arange(64), np.arange(64)[::-1].copy()):
        pool = make_pool(sh, 1, 512, "bf16", "bf16", sentinel_seed=9)
        for i, s in enumerate(slots):
            put_slot(pool, 0, int(s), w["ssm0"][i], w["conv0"][i])
        o = torch.from_numpy(order).cuda()
        y = torch.empty((64, sh.intermediate), dtype=torch.bfloat16, device="cuda")
        x, B, C = pool.split_xbc(u[o])
        pool.decode_step(0, W, torch.from_numpy(slots[order]).cuda(), x, B, C, z[o], dt[o], y)
        yy = torch.empty_like(y)
        yy[o] = y
        outs.append((yy.view(torch.int16).clone(), raw_bytes(pool.ssm), raw_bytes(pool.conv)))
        del pool
    for k in range(1, 3):
        for a, b in zip(outs[0], outs[k]):
            assert torch.equal(a, b)


def test_fp32_state_decode_at_8b_shape():
    """fp32 state, bf16 io, 32 sequences: the lane layout for 32-lane rows."""
    w = synth.decode_workload(11, batch=32, num_slots=40, ssm_dtype="f32", conv_dtype="bf16")
    sh, slots = w["shape"], w["slots"]
    pool = make_pool(sh, 1, 40, "f32", "bf16")
    for i, s in enumerate(slots):
        put_slot(pool, 0, int(s), w["ssm0"][i], w["conv0"][i])
    y = torch.empty((32, sh.intermediate), dtype=torch.float32, device="cuda")
    x, B, C = pool.split_xbc(dev(w["u"], "bf16"))
    pool.decode_step(0, weights(w["params"]), torch.from_numpy(slots).cuda(), x, B, C, dev(w["z"], "bf16"),
                     dev(w["dt"], "bf16"), y)
    ref = orc.PoolRef(sh, 1, 32, "f32", "bf16")
    ref.ssm[0], ref.conv[0] = w["ssm0"], w["conv0"]
    y_ref = orc.decode_step(ref, 0, w["params"], np.arange(32), w["u"], w["z"], w["dt"], "f32")
    assert rel_err(host(y), y_ref) <= TOL["f32"]
    for i, s in enumerate(slots):
        assert rel_err(host(pool.ssm[0, int(s)]), ref.ssm[0, i]) <= TOL["f32"]


# (heads, head_dim, d_state, groups, conv kernel): every supported d_state, head_dim other than 64,
# group counts other than a power of two, every conv width, and one group of 128 heads (a
# workgroup with 67.6 KB of LDS, above the default 64 KiB limit)
DECODE_SHAPES = [(4, 32, 32, 2, 2), (6, 64, 64, 3, 3), (4, 128, 256, 1, 4), (8, 16, 16, 4, 4), (128, 64, 128, 1, 4)]


@pytest.mark.parametrize("shape", DECODE_SHAPES, ids=lambda t: "H%dP%dN%dG%dW%d" % t)
@pytest.mark.parametrize("ssm_dtype", ["bf16", "f32"])
def test_decode_other_shapes(shape, ssm_dtype):
    sh = synth.Shape(*shape)
    rng = np.random.default_rng(500 + sum(shape))
    params = synth.layer_params(rng, sh)
    slots = np.array([6, 1, 9, 3, 12], np.int32)
    n = len(slots)
    io = ssm_dtype
    log(f"case: decode shape={shape} ssm={ssm_dtype}, {n} rows, 4 steps")
    ssm0 = synth.cast_exact(synth.normal(rng, (n, sh.nheads, sh.head_dim, sh.d_state), 0.1), ssm_dtype)
    conv0 = synth.cast_exact(synth.normal(rng, (n, sh.conv_dim, sh.conv_kernel - 1), 0.1), "bf16")
    pool = make_pool(sh, 1, 16, ssm_dtype, "bf16")
    ref = orc.PoolRef(sh, 1, 16, ssm_dtype, "bf16")
    for i, s in enumerate(slots):
        put_slot(pool, 0, int(s), ssm0[i], conv0[i])
        ref.ssm[0, s], ref.conv[0, s] = ssm0[i], conv0[i]
    before_s, before_c = raw_bytes(pool.ssm), raw_bytes(pool.conv)
    W = weights(params)
    sl = torch.from_numpy(slots).cuda()
    y = torch.empty((n, sh.intermediate), dtype=torch.float32 if io == "f32" else torch.bfloat16, device="cuda")
    for t in range(4):
        u, z, dt = synth._tokens(rng, sh, n, io)
        x, B, C = pool.split_xbc(dev(u, io))
        pool.decode_step(0, W, sl, x, B, C, dev(z, io), dev(dt, io), y, slots_host=slots)
        y_ref = orc.decode_step(ref, 0, params, slots, u, z, dt, io)
        assert rel_err(host(y), y_ref) <= TOL[ssm_dtype], t
    for i, s in enumerate(slots):
        assert rel_err(host(pool.ssm[0, s]), ref.ssm[0, s]) <= TOL[ssm_dtype]
        assert np.array_equal(host(pool.conv[0, s]), ref.conv[0, s])
    assert untouched(before_s, pool.ssm, slots) and untouched(before_c, pool.conv, slots)


def test_batch_above_the_grid_row_limit_is_split_into_launches():
    """70,000 rows (more than one launch's 65,535 grid rows): live rows on both sides of the split
    match the oracle; the padding rows between them are zero and touch nothing."""
    sh = synth.TINY
    rng = np.random.default_rng(6)
    params = synth.layer_params(rng, sh)
    pool = make_pool(sh, 1, 8, "f32", "f32")
    n = 70000
    live = {3: 1, 65534: 2, 65535: 5, 69999: 6}            # row -> slot
    slots = np.full(n, -1, np.int32)
    ref = orc.PoolRef(sh, 1, 8, "f32", "f32")
    for r, s in live.items():
        slots[r] = s
        st = synth.cast_exact(rng.normal(0, 0.1, (sh.nheads, sh.head_dim, sh.d_state)), "f32")
        cv = synth.cast_exact(rng.normal(0, 0.1, (sh.conv_dim, sh.conv_kernel - 1)), "f32")
        put_slot(pool, 0, s, st, cv)
        ref.ssm[0, s], ref.conv[0, s] = st, cv
    log(f"case: decode of {n} rows, {len(live)} live, TINY shape")
    before_s = raw_bytes(pool.ssm)
    u = torch.randn((n, sh.conv_dim), device="cuda")
    z = torch.randn((n, sh.intermediate), device="cuda")
    dt = torch.randn((n, sh.nheads), device="cuda")
    y = torch.full((n, sh.intermediate), 7.0, device="cuda")
    x, B, C = pool.split_xbc(u)
    pool.decode_step(0, weights(params), torch.from_numpy(slots).cuda(), x, B, C, z, dt, y, slots_host=slots)
    torch.cuda.synchronize()
    rows = sorted(live)
    y_ref = orc.decode_step(ref, 0, params, [live[r] for r in rows], host(u[rows]), host(z[rows]), host(dt[rows]),
                            "f32")
    assert rel_err(host(y[rows]), y_ref) <= TOL["f32"]
    pad = torch.ones(n, dtype=torch.bool, device="cuda")
    pad[rows] = False
    assert not bool(y[pad].any())
    for r in rows:
        s = live[r]
        assert rel_err(host(pool.ssm[0, s]), ref.ssm[0, s]) <= TOL["f32"]
        assert np.array_equal(host(pool.conv[0, s]), ref.conv[0, s])
    assert untouched(before_s, pool.ssm, list(live.values()))
