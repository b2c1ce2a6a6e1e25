"""GPU checks of the state-only families, GDN and KDA, on pools laid out as the MambaSpec table
of the study notes gives them (GDN: (num_v_heads, head_v_dim, head_k_dim) bf16; KDA:
(num_heads, head_dim, head_dim) fp32, conv window bf16): the slot copy bit for bit, and the int8
store's codes, scales and restored states bit for bit against the oracle.  The pages give no
recurrence for either family, so nothing else runs on these pools."""
import numpy as np
import pytest
import torch

from oracle import mamba2 as orc
from recurrent_state_update_amd import synth
from recurrent_state_update_amd.pool import Pool
from tests.gpu_helpers import host, log, raw_bytes, untouched

pytestmark = pytest.mark.gpu

# (family, nheads, head_dim, d_state, n_groups): GDN as (Hv, dv, dk, Hk), KDA as (H, d, d, H)
SMALL = [("GDN", 8, 64, 32, 2), ("KDA", 4, 64, 64, 4)]
WIDE = [("GDN", 32, 128, 128, 16), ("KDA", 32, 128, 128, 32)]


def _pool(family, H, P, N, G, L, S, seed, W=4):
    pool = (Pool.allocate_gdn(L, S, H, P, N, G, W) if family == "GDN" else Pool.allocate_kda(L, S, H, P, W))
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    for t in (pool.ssm, pool.conv):
        b = t.view(torch.uint8)
        b.copy_(torch.randint(0, 256, b.shape, generator=g, device="cuda", dtype=torch.int32).to(torch.uint8))
    return pool


def _i32(v):
    return torch.tensor(v, dtype=torch.int32, device="cuda")


@pytest.mark.parametrize("case", SMALL + WIDE, ids=lambda c: f"{c[0]}-{c[1]}x{c[2]}x{c[3]}")
@pytest.mark.parametrize("layer", [-1, 1])
def test_slot_copy_is_bit_exact(case, layer):
    family, H, P, N, G = case
    L, S = 3, 9
    log(f"case: {family} slot copy H={H} P={P} N={N} layer={layer}")
    pool = _pool(family, H, P, N, G, L, S, seed=31)
    bs, bc = raw_bytes(pool.ssm), raw_bytes(pool.conv)
    src_h, dst_h = [0, 4, 7], [8, 2, 5]
    pool.checkpoint(layer, _i32(src_h), _i32(dst_h), src_host=src_h, dst_host=dst_h)
    torch.cuda.synchronize()
    layers = range(L) if layer < 0 else [layer]
    for l in layers:
        for s, d in zip(src_h, dst_h):
            assert torch.equal(pool.ssm[l, d].view(torch.uint8).reshape(-1), bs.view(L, S, -1)[l, s])
            assert torch.equal(pool.conv[l, d].view(torch.uint8).reshape(-1), bc.view(L, S, -1)[l, s])
    only = None if layer < 0 else layer
    assert untouched(bs, pool.ssm, dst_h, layer=only) and untouched(bc, pool.conv, dst_h, layer=only)


@pytest.mark.parametrize("case", SMALL + WIDE, ids=lambda c: f"{c[0]}-{c[1]}x{c[2]}x{c[3]}")
def test_int8_store_matches_the_oracle_bit_for_bit(case):
    family, H, P, N, G = case
    L, S, E = 2, 8, 4
    ssm_dt = "bf16" if family == "GDN" else "f32"
    log(f"case: {family} int8 store H={H} P={P} N={N}")
    sh = synth.Shape(H, P, N, G, 4)
    pool = _pool(family, H, P, N, G, L, S, seed=41)
    ref = orc.PoolRef(sh, L, S, ssm_dt, "bf16")
    rng = np.random.default_rng(42)
    src = [1, 6, 3]
    for l in range(L):
        for s in src:
            st = synth.cast_exact(rng.normal(0, 0.1, (H, P, N)), ssm_dt)
            st[0, :, 1] = 0.0                          # a zero column: scale 0, codes 0
            cv = synth.cast_exact(rng.normal(0, 0.1, (sh.conv_dim, 3)), "bf16")
            pool.ssm[l, s] = torch.from_numpy(st).to(pool.ssm.dtype).cuda()
            pool.conv[l, s] = torch.from_numpy(cv).to(pool.conv.dtype).cuda()
            ref.ssm[l, s], ref.conv[l, s] = st, cv
    store = pool.int8_store(E)
    sref = orc.Int8StoreRef(ref, E)
    ent = [2, 0, 3]
    pool.int8_put(store, -1, _i32(src), _i32(ent), slots_host=src, entries_host=ent)
    torch.cuda.synchronize()
    orc.int8_store_put(ref, sref, -1, src, ent)
    codes, scales = store.codes.cpu().numpy(), store.scales.cpu().numpy()
    for e in ent:
        assert np.array_equal(codes[e], sref.codes[e]), e
        assert np.array_equal(scales[e].view(np.uint32), sref.scales[e].view(np.uint32)), e
        assert np.array_equal(host(store.conv[e]), sref.conv[e]), e
    dst, back = [0, 5], [0, 3]
    bs, bc = raw_bytes(pool.ssm), raw_bytes(pool.conv)
    pool.int8_get(store, -1, _i32(back), _i32(dst), entries_host=back, slots_host=dst)
    torch.cuda.synchronize()
    orc.int8_store_get(sref, ref, -1, back, dst)
    for l in range(L):
        for s in dst:
            assert np.array_equal(host(pool.ssm[l, s]), ref.ssm[l, s]), (l, s)
            assert np.array_equal(host(pool.conv[l, s]), ref.conv[l, s]), (l, s)
    assert untouched(bs, pool.ssm, dst) and untouched(bc, pool.conv, dst)
