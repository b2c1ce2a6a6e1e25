"""GPU checks of the slot-to-slot checkpoint copy (bit-exact placement)."""
import numpy as np
import pytest
import torch

from recurrent_state_update_amd import synth
from tests.gpu_helpers import log, make_pool, raw_bytes, untouched

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("ssm_dtype,layer", [("bf16", 1), ("f32", -1)])
def test_copy_is_bit_exact_and_touches_only_destinations(ssm_dtype, layer):
    sh = synth.NEMOTRON_H
    log(f"case: checkpoint copy ssm={ssm_dtype} layer={layer}")
    pool = make_pool(sh, 3, 12, ssm_dtype, "bf16", sentinel_seed=21)
    src_h, dst_h = [0, 5, 7], [3, 11, 2]
    before_s, before_c = raw_bytes(pool.ssm), raw_bytes(pool.conv)
    src = torch.tensor(src_h, dtype=torch.int32, device="cuda")
    dst = torch.tensor(dst_h, dtype=torch.int32, device="cuda")
    pool.checkpoint(layer, src, dst, src_host=src_h, dst_host=dst_h)
    torch.cuda.synchronize()
    layers = range(3) if layer < 0 else [layer]
    bs = before_s.view(3, 12, -1)
    bc = before_c.view(3, 12, -1)
    for l in layers:
        for s, d in zip(src_h, dst_h):
            assert torch.equal(pool.ssm[l, d].view(torch.uint8).reshape(-1), bs[l, s])
            assert torch.equal(pool.conv[l, d].view(torch.uint8).reshape(-1), bc[l, s])
    # nothing else changed: other layers entirely, other slots of the copied layers
    L, S = 3, 12
    mask = torch.ones((L, S), dtype=torch.bool, device="cuda")
    for l in layers:
        for d in dst_h:
            mask[l, d] = False
    assert torch.equal(pool.ssm.view(torch.uint8).view(L, S, -1)[mask], bs[mask])
    assert torch.equal(pool.conv.view(torch.uint8).view(L, S, -1)[mask], bc[mask])


def test_copy_skips_out_of_range_pairs_on_device():
    sh = synth.TINY
    pool = make_pool(sh, 1, 8, "f32", "f32", sentinel_seed=22)
    before_s, before_c = raw_bytes(pool.ssm), raw_bytes(pool.conv)
    src = torch.tensor([1, 40, 2], dtype=torch.int32, device="cuda")
    dst = torch.tensor([-3, 4, 6], dtype=torch.int32, device="cuda")
    pool.checkpoint(0, src, dst)
    torch.cuda.synchronize()
    b = lambda t: t.view(torch.uint8)
    assert torch.equal(b(pool.ssm[0, 6]), b(pool.ssm[0, 2])) and torch.equal(b(pool.conv[0, 6]), b(pool.conv[0, 2]))
    assert untouched(before_s, pool.ssm, [6]) and untouched(before_c, pool.conv, [6])
