"""GPU checks of the int8 checkpoint store against the oracle: codes and scales bit-exact (both
sides decide them in fp32), restored states bit-exact, placement exact, and a prefill that
continues from a restored state within the oracle tolerance."""
import numpy as np
import pytest
import torch

from oracle import mamba2 as orc
from recurrent_state_update_amd import synth
from tests.gpu_helpers import TOL, dev, host, log, make_pool, put_slot, raw_bytes, rel_err, untouched, weights

pytestmark = pytest.mark.gpu


def _states(rng, n, sh, ssm_dtype):
    """Seeded N(0, 0.1) states with edge columns: all zero, one large value, all negative."""
    s = rng.normal(0, 0.1, (n, sh.nheads, sh.head_dim, sh.d_state))
    s[0, 0, :, 3] = 0.0
    s[0, 1, :, 5] = 0.0
    s[0, 1, 2, 5] = 7.25
    s[-1, -1, :, 0] = -np.abs(s[-1, -1, :, 0])
    return synth.cast_exact(s, ssm_dtype)


def _fill_random(t, seed):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    b = t.view(torch.uint8)
    b.copy_(torch.randint(0, 256, b.shape, generator=g, device="cuda", dtype=torch.int32).to(torch.uint8))


def _i32(v):
    return torch.tensor(v, dtype=torch.int32, device="cuda")


@pytest.mark.parametrize("ssm_dtype,layer,sh", [
    ("bf16", -1, synth.Shape(4, 32, 64, 2, 4)), ("f32", 1, synth.Shape(4, 32, 64, 2, 4)),
    ("bf16", 0, synth.Shape(4, 32, 64, 2, 4)),
    ("f32", -1, synth.Shape(2, 128, 256, 1, 3)),    # 128 rows of 256: more rows than a thread holds
    ("bf16", 0, synth.Shape(3, 24, 40, 3, 2)),      # d_state 40: 5 column groups, ragged row groups
], ids=["bf16-all", "f32-layer1", "bf16-layer0", "f32-tall", "bf16-ragged"])
def test_put_and_get_match_the_oracle_bit_for_bit(ssm_dtype, layer, sh):
    L, S, E = 2, 12, 5
    log(f"case: int8 store {ssm_dtype} layer={layer}")
    rng = np.random.default_rng(60)
    pool = make_pool(sh, L, S, ssm_dtype, "bf16", sentinel_seed=61)
    ref = orc.PoolRef(sh, L, S, ssm_dtype, "bf16")
    src = [1, 4, 7]
    for l in range(L):
        st = _states(rng, len(src), sh, ssm_dtype)
        cv = synth.cast_exact(rng.normal(0, 0.1, (len(src), sh.conv_dim, sh.conv_kernel - 1)), "bf16")
        for i, s in enumerate(src):
            put_slot(pool, l, s, st[i], cv[i])
            ref.ssm[l, s], ref.conv[l, s] = st[i], cv[i]
    store = pool.int8_store(E)
    for i, t in enumerate((store.codes, store.scales, store.conv)):
        _fill_random(t, 70 + i)
    sref = orc.Int8StoreRef(ref, E)
    before = [raw_bytes(t) for t in (store.codes, store.scales, store.conv)]
    ent = [0, 3, 2]
    pool.int8_put(store, layer, _i32(src), _i32(ent), slots_host=src, entries_host=ent)
    torch.cuda.synchronize()
    orc.int8_store_put(ref, sref, layer, src, ent)
    layers = range(L) if layer < 0 else [layer]
    codes, scales = store.codes.cpu().numpy(), store.scales.cpu().numpy()
    for e in ent:
        for l in layers:
            assert np.array_equal(codes[e, l], sref.codes[e, l]), (e, l)
            assert np.array_equal(scales[e, l].view(np.uint32), sref.scales[e, l].view(np.uint32)), (e, l)
            assert np.array_equal(host(store.conv[e, l]), sref.conv[e, l]), (e, l)
    written = {(e, l) for e in ent for l in layers}
    for t, b in zip((store.codes, store.scales, store.conv), before):
        for e in range(E):
            for l in range(L):
                if (e, l) not in written:
                    assert torch.equal(t[e, l].view(torch.uint8).reshape(-1), b.view(E, L, -1)[e, l])
    # restore two entries into fresh slots
    dst, back = [9, 10], [3, 0]
    bs, bc = raw_bytes(pool.ssm), raw_bytes(pool.conv)
    pool.int8_get(store, layer, _i32(back), _i32(dst), entries_host=back, slots_host=dst)
    torch.cuda.synchronize()
    orc.int8_store_get(sref, ref, layer, back, dst)
    for l in layers:
        for s in dst:
            assert np.array_equal(host(pool.ssm[l, s]), ref.ssm[l, s]), (l, s)
            assert np.array_equal(host(pool.conv[l, s]), ref.conv[l, s])
    live = [(l, s) for l in layers for s in dst]
    for t, b in ((pool.ssm, bs), (pool.conv, bc)):
        for l in range(L):
            keep = [s for s in range(S) if (l, s) not in live]
            view = b.view(L, S, -1)
            for s in keep:
                assert torch.equal(t[l, s].view(torch.uint8).reshape(-1), view[l, s])
    # the restored state is within half a quantization step of the original (e.g. slot 4 -> entry 3 -> 9)
    for l in layers:
        amax = np.max(np.abs(ref.ssm[l, 4]), axis=1)
        err = np.abs(ref.ssm[l, 9] - ref.ssm[l, 4])
        tol = amax[:, None, :] / 254 * (1 + 2.0 ** -20) + np.abs(ref.ssm[l, 4]).max() * 2.0 ** -7
        assert np.all(err <= tol)


def test_out_of_range_device_pairs_are_skipped():
    sh = synth.TINY
    pool = make_pool(sh, 1, 6, "f32", "f32", sentinel_seed=62)
    rng = np.random.default_rng(63)
    put_slot(pool, 0, 2, _states(rng, 1, sh, "f32")[0], rng.normal(0, 0.1, (sh.conv_dim, sh.conv_kernel - 1)))
    store = pool.int8_store(3)
    for i, t in enumerate((store.codes, store.scales, store.conv)):
        _fill_random(t, 80 + i)
    before = [raw_bytes(t) for t in (store.codes, store.scales, store.conv)]
    pool.int8_put(store, 0, _i32([2, 9, 2]), _i32([-1, 0, 5]))     # every pair has an index out of range
    torch.cuda.synchronize()
    for t, b in zip((store.codes, store.scales, store.conv), before):
        assert torch.equal(t.view(torch.uint8).reshape(-1), b.reshape(-1))
    bs = raw_bytes(pool.ssm)
    pool.int8_get(store, 0, _i32([0, 7]), _i32([8, 1]))
    torch.cuda.synchronize()
    assert untouched(bs, pool.ssm, [])


def test_layer_shape_store_of_256_slots_sampled_against_the_oracle():
    """The Nemotron-H layer shape at the size the benchmark times (256 slots of a 512-slot bf16
    pool into 256 entries and back): codes and scales of sampled heads bit-exact, every column's
    largest code +-127, every restored value within half a step."""
    sh = synth.NEMOTRON_H
    log("case: int8 store, 256 slots, Nemotron-H layer shape")
    g = torch.Generator(device="cuda")
    g.manual_seed(90)
    pool = make_pool(sh, 1, 512, "bf16", "bf16", sentinel_seed=91)
    slots = torch.randperm(512, generator=g, device="cuda")[:256].to(torch.int32)
    pool.ssm[0, slots.long()] = (torch.randn((256,) + tuple(pool.ssm.shape[2:]), generator=g, device="cuda")
                                 * 0.1).bfloat16()
    pool.conv[0, slots.long()] = torch.randn((256,) + tuple(pool.conv.shape[2:]), generator=g,
                                             device="cuda").bfloat16()
    store = pool.int8_store(256)
    ent = torch.arange(256, dtype=torch.int32, device="cuda")
    pool.int8_put(store, 0, slots, ent)
    dst = torch.arange(256, 512, dtype=torch.int32, device="cuda")
    src_state = pool.ssm[0, slots.long()].clone()
    src_conv = pool.conv[0, slots.long()].clone()
    pool.int8_get(store, 0, ent, dst)
    torch.cuda.synchronize()
    codes = store.codes[:, 0].to(torch.int32)
    assert int(codes.abs().amax(dim=2).min()) == 127              # every column reaches +-127
    for e, h in [(0, 0), (17, 45), (128, 127), (255, 64)]:
        q, s = orc.int8_quantize(host(src_state[e, h]))
        assert np.array_equal(store.codes[e, 0, h].cpu().numpy(), q)
        assert np.array_equal(store.scales[e, 0, h].cpu().numpy().view(np.uint32), s.view(np.uint32))
        assert np.array_equal(host(pool.ssm[0, 256 + e, h]), orc.int8_dequantize(q, s, "bf16"))
    x = src_state.float()
    step = x.abs().amax(dim=2, keepdim=True) / 127
    err = (pool.ssm[0, 256:].float() - x).abs()
    assert bool((err <= step / 2 * (1 + 2.0 ** -20) + x.abs() * 2.0 ** -8).all())
    assert torch.equal(pool.conv[0, 256:], src_conv)


def test_prefill_continues_from_a_restored_state_like_the_oracle():
    """A slot restored from the int8 store seeds a prefill of 300 tokens that matches the oracle
    run from the oracle's restored state."""
    sh = synth.Shape(8, 64, 128, 2, 4)
    rng = np.random.default_rng(95)
    params, ssm0, conv0, u, z, dt = synth.random_problem(rng, sh, 300, "bf16")
    ssm0, conv0 = synth.cast_exact(ssm0, "bf16"), synth.cast_exact(conv0, "bf16")
    pool = make_pool(sh, 1, 6, "bf16", "bf16", sentinel_seed=96)
    ref = orc.PoolRef(sh, 1, 6, "bf16", "bf16")
    put_slot(pool, 0, 1, ssm0, conv0)
    ref.ssm[0, 1], ref.conv[0, 1] = ssm0, conv0
    store = pool.int8_store(2)
    sref = orc.Int8StoreRef(ref, 2)
    pool.int8_put(store, 0, _i32([1]), _i32([1]))
    pool.int8_get(store, 0, _i32([1]), _i32([4]))
    orc.int8_store_put(ref, sref, 0, [1], [1])
    orc.int8_store_get(sref, ref, 0, [1], [4])
    W = weights(params)
    y = torch.empty((300, sh.intermediate), dtype=torch.bfloat16, device="cuda")
    x, B, C = pool.split_xbc(dev(u, "bf16"))
    pool.prefill(0, W, np.array([0, 300], np.int32), [4], [1], x, B, C, dev(z, "bf16"), dev(dt, "bf16"), y,
                 chunk_size=64)
    torch.cuda.synchronize()
    y_ref = orc.prefill(ref, 0, params, [0, 300], [4], [1], [0], u, z, dt, "bf16")
    e = rel_err(host(y), y_ref)
    log(f"y rel error after restore {e:.3e}")
    assert e <= TOL["bf16"]
    assert rel_err(host(pool.ssm[0, 4]), ref.ssm[0, 4]) <= TOL["bf16"]
    assert np.array_equal(host(pool.conv[0, 4]), ref.conv[0, 4])
