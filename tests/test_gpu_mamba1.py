"""GPU parity of the Mamba1 decode step and prefill (the pool's second state family) against the oracle."""
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


def _m1_prefill_case(D, N, W, ssm_dtype, Q, lens, has_init, start_pos, interval, ck, seed, L=2, S=16,
                     layer=1, slots=None, draw_rows=0, io=None):
    """Run one Mamba1 prefill on the GPU and on the oracle from the same seeded pool and rows."""
    rng = np.random.default_rng(seed)
    params = synth.mamba1_layer_params(rng, D, N, W)
    ns = len(lens)
    slots = np.arange(ns, dtype=np.int32)[::-1].copy() + 3 if slots is None else np.asarray(slots, np.int32)
    pool = _pool(D, N, W, L, S, ssm_dtype, "bf16", seed + 1)
    ref = orc.Mamba1PoolRef(D, N, W, L, S, ssm_dtype, "bf16")
    for s in range(S):          # every slot holds a state; the oracle mirrors the live ones
        h0 = synth.cast_exact(rng.normal(0, 0.1, (D, N)), ssm_dtype)
        w0 = synth.cast_exact(rng.normal(0, 0.1, (D, W - 1)), "bf16")
        pool.ssm[layer, s, :, 0] = torch.from_numpy(h0).to(TD[ssm_dtype]).cuda()
        pool.conv[layer, s] = torch.from_numpy(w0).to(torch.bfloat16).cuda()
        ref.ssm[layer, s], ref.conv[layer, s] = h0, w0
    before_s, before_c = _raw(pool.ssm), _raw(pool.conv)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T = int(cu[-1])
    io = io or ssm_dtype
    x, z, dt, Bm, Cm = (r[:T] for r in synth.mamba1_tokens(rng, max(T, draw_rows), D, N, io))
    y = torch.full((T, D), float("nan"), dtype=TD[ssm_dtype], device="cuda")
    pool.mamba1_prefill(layer, weights(params), cu, slots, has_init, dev(x, io), dev(Bm, io), dev(Cm, io),
                        dev(z, io), dev(dt, io), y, start_pos=start_pos, chunk_size=Q, ckpt_interval=interval,
                        ckpt_slots=ck)
    y_ref = orc.mamba1_prefill(ref, layer, params, cu, slots, has_init, start_pos, x, z, dt, Bm, Cm, ssm_dtype,
                               ckpt_interval=interval, ckpt_slots=ck)
    return pool, ref, host(y), y_ref, before_s, before_c


@pytest.mark.parametrize("D,N,W,ssm_dtype,Q", [(64, 16, 4, "bf16", 32), (64, 16, 4, "f32", 16),
                                               (48, 8, 2, "f32", 64), (32, 64, 3, "bf16", 48),
                                               (16, 256, 4, "f32", 256)])
def test_mamba1_prefill_matches_the_oracle(D, N, W, ssm_dtype, Q):
    """Ragged batch (an empty sequence, one row, sequences across several chunks and a tail),
    seeded and zero starts, nonzero start positions, checkpoints every 24 positions (off the chunk
    grid) with a skipped entry: outputs, final and checkpoint states against the oracle, windows
    exact, every other slot and layer untouched."""
    lens = [0, 1, 37, 200, 64, 130]
    has_init = [1, 1, 0, 1, 0, 1]
    start_pos = np.array([0, 7, 0, 40, 0, 5], np.int32)
    ck = np.full((6, 9), -1, np.int32)
    ck[3] = [0, 1, -1, 15, 14, 13, -1, -1, 12]      # positions 48 .. 240 of sequence 3, some skipped
    ck[4, :2] = [2, 11]                               # positions 24 and 48 of sequence 4 (its last row)
    ck[5, :5] = [10, -1, 9, -1, -1]                   # positions 24 .. 120 of sequence 5
    log(f"case: Mamba1 prefill D={D} N={N} W={W} ssm={ssm_dtype} Q={Q} lens={lens}")
    slots = np.array([3, 4, 5, 6, 7, 8], np.int32)
    pool, ref, y, y_ref, before_s, before_c = _m1_prefill_case(D, N, W, ssm_dtype, Q, lens, has_init, start_pos,
                                                               24, ck, 900 + N + Q, slots=slots)
    err = rel_err(y, y_ref)
    log(f"max rel y error: {err:.3e}")
    assert err <= TOL[ssm_dtype]
    written = set(int(s) for s, n in zip(slots, lens) if n > 0)
    for s, n in zip(slots, lens):
        if n > 0:
            assert rel_err(host(pool.ssm[1, s, :, 0]), ref.ssm[1, s]) <= TOL[ssm_dtype]
            assert np.array_equal(host(pool.conv[1, s]), ref.conv[1, s])
    for si in range(6):
        p0, n = int(start_pos[si]), lens[si]
        for k in range(ck.shape[1]):
            p = (p0 // 24 + 1 + k) * 24
            if ck[si, k] >= 0 and p <= p0 + n:
                c = int(ck[si, k])
                written.add(c)
                assert rel_err(host(pool.ssm[1, c, :, 0]), ref.ssm[1, c]) <= TOL[ssm_dtype], (si, k)
                assert np.array_equal(host(pool.conv[1, c]), ref.conv[1, c]), (si, k)
    assert written == {0, 1, 2, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15}
    live = torch.zeros((2, 16), dtype=torch.bool, device="cuda")
    live[1, sorted(written)] = True
    for t, b in ((pool.ssm, before_s), (pool.conv, before_c)):
        assert torch.equal(t.view(torch.uint8).view(2, 16, -1)[~live], b.view(2, 16, -1)[~live])


@pytest.mark.parametrize("ssm_dtype,io", [("f32", "bf16"), ("bf16", "f32")])
def test_mamba1_prefill_with_rows_in_the_other_dtype(ssm_dtype, io):
    """Rows in bf16 with an fp32 state and the reverse (y in the state dtype): outputs, final and
    checkpoint states against the oracle."""
    D, N, W = 64, 32, 4
    lens = [90, 1, 40]
    ck = np.array([[9, 10, -1], [-1, -1, -1], [11, -1, -1]], np.int32)
    log(f"case: Mamba1 prefill ssm={ssm_dtype} io={io}")
    pool, ref, y, y_ref, _, _ = _m1_prefill_case(D, N, W, ssm_dtype, 32, lens, [1, 0, 1],
                                                 np.array([0, 3, 0], np.int32), 32, ck, 940, io=io)
    assert rel_err(y, y_ref) <= TOL[ssm_dtype]
    for s in (3, 4, 5, 9, 10, 11):
        assert rel_err(host(pool.ssm[1, s, :, 0]), ref.ssm[1, s]) <= TOL[ssm_dtype], s
        assert np.array_equal(host(pool.conv[1, s]), ref.conv[1, s]), s


def test_mamba1_prefill_chunk_size_and_batch_invariance():
    """A sequence's outputs and states do not depend on its batch neighbours (bit for bit) and
    agree across chunk sizes 16 and 512 to the fp32 tolerance."""
    D, N, W = 128, 16, 4
    lens = [300, 77, 1, 129]
    has = [1, 0, 1, 1]
    sp = np.array([3, 0, 9, 0], np.int32)
    runs = {}
    for Q in (16, 512):
        pool, _, y, _, _, _ = _m1_prefill_case(D, N, W, "f32", Q, lens, has, sp, 0, None, 950)
        runs[Q] = (y, host(pool.ssm[1, :, :, 0]), host(pool.conv[1]))
    assert rel_err(runs[16][0], runs[512][0]) <= TOL["f32"]
    assert rel_err(runs[16][1], runs[512][1]) <= TOL["f32"]
    assert np.array_equal(runs[16][2], runs[512][2])
    # sequence 0 alone: same slot, same starting pool, same rows
    pool, _, y0, _, _, _ = _m1_prefill_case(D, N, W, "f32", 16, lens[:1], has[:1], sp[:1], 0, None, 950,
                                            slots=[6], draw_rows=sum(lens))
    assert np.array_equal(y0, runs[16][0][:300])
    assert np.array_equal(host(pool.ssm[1, 6, :, 0]), runs[16][1][6])


def test_mamba1_prefill_then_decode_continues_the_sequence():
    """Prefill of 90 rows then 10 decode steps equals the oracle's 100-row prefill's last outputs
    and final state (fp32 pool, so nothing is rounded at the hand-over)."""
    D, N, W = 64, 32, 4
    rng = np.random.default_rng(960)
    params = synth.mamba1_layer_params(rng, D, N, W)
    pool = _pool(D, N, W, 1, 4, "f32", "f32", 961)
    ref = orc.Mamba1PoolRef(D, N, W, 1, 4, "f32", "f32")
    x, z, dt, Bm, Cm = synth.mamba1_tokens(rng, 100, D, N, "f32")
    y_ref = orc.mamba1_prefill(ref, 0, params, [0, 100], [2], [0], None, x, z, dt, Bm, Cm, "f32")
    W_ = weights(params)
    y = torch.empty((90, D), dtype=torch.float32, device="cuda")
    pool.mamba1_prefill(0, W_, [0, 90], [2], [0], dev(x[:90], "f32"), dev(Bm[:90], "f32"), dev(Cm[:90], "f32"),
                        dev(z[:90], "f32"), dev(dt[:90], "f32"), y, chunk_size=32)
    assert rel_err(host(y), y_ref[:90]) <= TOL["f32"]
    sl = torch.tensor([2], dtype=torch.int32, device="cuda")
    yd = torch.empty((1, D), dtype=torch.float32, device="cuda")
    for t in range(90, 100):
        r = slice(t, t + 1)
        pool.mamba1_decode_step(0, W_, sl, dev(x[r], "f32"), dev(Bm[r], "f32"), dev(Cm[r], "f32"),
                                dev(z[r], "f32"), dev(dt[r], "f32"), yd, slots_host=[2])
        assert rel_err(host(yd)[0], y_ref[t]) <= TOL["f32"], t
    assert rel_err(host(pool.ssm[0, 2, :, 0]), ref.ssm[0, 2]) <= TOL["f32"]
    assert np.array_equal(host(pool.conv[0, 2]), ref.conv[0, 2])    # windows are copies: bit for bit


def test_mamba1_prefill_at_the_7b_width():
    """D = 8192, N = 16, W = 4, bf16 pool and rows, chunk 256: four sequences (1024 rows) with
    checkpoints every 256 positions, against the oracle."""
    D, N, W = synth.MAMBA1_D, synth.MAMBA1_N, synth.MAMBA1_W
    lens = [512, 300, 1, 211]
    ck = np.array([[8, 9], [10, -1], [-1, -1], [-1, -1]], np.int32)
    log(f"case: Mamba1 prefill D={D} N={N}, lens {lens}")
    pool, ref, y, y_ref, _, _ = _m1_prefill_case(D, N, W, "bf16", 256, lens, [1, 0, 1, 1],
                                                 np.array([0, 0, 5, 100], np.int32), 256, ck, 970, L=1, S=12,
                                                 layer=0, slots=[0, 1, 2, 3])
    err = rel_err(y, y_ref)
    log(f"max rel y error: {err:.3e}")
    assert err <= TOL["bf16"]
    for s in (0, 1, 2, 3, 8, 9, 10):
        assert rel_err(host(pool.ssm[0, s, :, 0]), ref.ssm[0, s]) <= TOL["bf16"], s
        assert np.array_equal(host(pool.conv[0, s]), ref.conv[0, s]), s


@pytest.mark.parametrize("lens", [[1024, 1024, 1024, 1024, 700, 1, 1300, 45], [2000, 1]])
def test_mamba1_prefill_with_the_library_chunking(lens):
    """chunk_size 0 at D = 8192, N = 16, bf16: eight sequences (128 workgroups each: chunks of
    about total/8 = 768 rows, so the longer sequences are cut in two) and two (cut into 256-row
    chunks to fill the GPU), seeded and zero starts, checkpoints every 300 positions, against the
    oracle."""
    D, N, W = synth.MAMBA1_D, synth.MAMBA1_N, synth.MAMBA1_W
    ns = len(lens)
    ck = np.full((ns, 7), -1, np.int32)
    ck[0, :3] = [8, 9, 10]
    if ns > 2:
        ck[6, :1] = [11]
    log(f"case: Mamba1 prefill D={D} N={N}, library chunking, lens {lens}")
    has = [1, 0] * (ns // 2)
    sp = np.array([0, 10] * (ns // 2), np.int32)
    pool, ref, y, y_ref, _, _ = _m1_prefill_case(D, N, W, "bf16", 0, lens, has, sp, 300, ck, 975 + ns, L=1,
                                                 S=12, layer=0, slots=list(range(ns)))
    err = rel_err(y, y_ref)
    log(f"max rel y error: {err:.3e}")
    assert err <= TOL["bf16"]
    for s in list(range(ns)) + [8, 9, 10, 11]:
        if s >= 8 and not (ck == s).any():
            continue
        assert rel_err(host(pool.ssm[0, s, :, 0]), ref.ssm[0, s]) <= TOL["bf16"], s
        assert np.array_equal(host(pool.conv[0, s]), ref.conv[0, s]), s


@pytest.mark.parametrize("Q", [0, 16])
def test_mamba1_prefill_checkpoint_at_every_row(Q):
    """Checkpoint interval 1: a state after every row, so checkpoints fall on every position of the
    kernel's 4-row groups and on the last real row before a padded group (lengths 5 and 11, start
    positions 0 and 2, fp32 state, one sequence seeded): every checkpoint state against the oracle,
    every window bit for bit."""
    D, N, W = 64, 16, 4
    lens = [5, 11]
    ck = np.full((2, 11), -1, np.int32)
    ck[0, :5] = np.arange(2, 7)
    ck[1, :11] = np.arange(7, 18)
    log(f"case: Mamba1 prefill Q={Q}, checkpoint every row, lens {lens}")
    pool, ref, y, y_ref, _, _ = _m1_prefill_case(D, N, W, "f32", Q, lens, [1, 0], np.array([0, 2], np.int32), 1,
                                                 ck, 996, L=1, S=18, layer=0, slots=[0, 1])
    assert rel_err(y, y_ref) <= TOL["f32"]
    for s in range(18):
        assert rel_err(host(pool.ssm[0, s, :, 0]), ref.ssm[0, s]) <= TOL["f32"], s
        assert np.array_equal(host(pool.conv[0, s]), ref.conv[0, s]), s


def test_mamba1_prefill_at_the_largest_chunk_size():
    """chunk_size 4096 (the upper bound): a 5000-row sequence (two chunks, the second partial) and a
    4096-row one (one full chunk), seeded, with checkpoints every 1000 positions, against the oracle."""
    D, N, W = 32, 16, 4
    lens = [5000, 4096]
    ck = np.full((2, 6), -1, np.int32)
    ck[0, :5] = [8, 9, 10, 11, 12]                    # positions 1000 .. 5000 of sequence 0
    ck[1, :4] = [13, 14, 15, 2]                       # positions 1000 .. 4000 of sequence 1
    log("case: Mamba1 prefill chunk 4096, lens 5000 and 4096")
    pool, ref, y, y_ref, _, _ = _m1_prefill_case(D, N, W, "f32", 4096, lens, [1, 1], np.array([0, 0], np.int32),
                                                 1000, ck, 990, L=1, S=16, layer=0, slots=[0, 1])
    assert rel_err(y, y_ref) <= TOL["f32"]
    for s in (0, 1, 2, 8, 9, 10, 11, 12, 13, 14, 15):
        assert rel_err(host(pool.ssm[0, s, :, 0]), ref.ssm[0, s]) <= TOL["f32"], s
        assert np.array_equal(host(pool.conv[0, s]), ref.conv[0, s]), s
