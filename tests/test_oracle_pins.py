"""Pins of the CPU oracle against what the pages and the mathematics fix.

Every test here runs on the CPU.  The oracle is checked against forms that do
not share its code path: the semiseparable matrix form built from explicit
products, a closed form for constant inputs, scipy's IIR filter, numpy's
convolution, torch's bf16 casts, and numbers printed on the pages
(tests/golden/*.json, each entry with its citation).
"""
import json
import math
import os

import numpy as np
import pytest
import scipy.signal
import scipy.special
import torch

from oracle import mamba2 as orc
from recurrent_state_update_amd import synth


def rel_err(a, b):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


# ---------------------------------------------------------------- rounding
def test_bf16_rounding_matches_torch_cast():
    rng = np.random.default_rng(123)
    n = 1_000_000
    mags = 10.0 ** rng.uniform(-42, 39, n)
    vals = rng.choice([-1.0, 1.0], n) * mags
    one = 1.0
    edges = np.array([
        0.0, -0.0, np.inf, -np.inf, np.nan,
        np.finfo(np.float32).max, -np.finfo(np.float32).max, 3.3895313892515355e38,
        np.finfo(np.float32).tiny, 1e-45, -1e-45, 1e-40,
        one + 2.0 ** -8, one + 3 * 2.0 ** -8, one + 2.0 ** -8 + 2.0 ** -30,  # ties and near-ties
        -(one + 2.0 ** -8), 2.0 ** 127 * (2 - 2.0 ** -8),
    ])
    vals = np.concatenate([vals, edges, rng.standard_normal(10000)])
    mine = orc.round_to(vals, "bf16")
    ref = torch.from_numpy(vals).to(torch.float32).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(mine, ref, equal_nan=True)
    finite = ~np.isnan(ref)                     # torch canonicalises NaN to 0xFFFF; NaN sign is free
    assert np.array_equal(np.signbit(mine[finite]), np.signbit(ref[finite]))
    # fp32 rounding against torch's cast as well
    ref32 = torch.from_numpy(vals).to(torch.float32).to(torch.float64).numpy()
    assert np.array_equal(orc.round_to(vals, "f32"), ref32, equal_nan=True)


# ---------------------------------------------------------------- elementwise
def test_softplus_and_silu_match_library_forms():
    v = np.concatenate([np.linspace(-60, 60, 20001), [-700.0, 700.0, 0.0]])
    assert np.allclose(orc.softplus(v), np.logaddexp(0.0, v), rtol=1e-14, atol=0)
    assert np.allclose(orc.silu(v), v * scipy.special.expit(v), rtol=1e-14, atol=1e-300)


# ---------------------------------------------------------------- conv
def test_conv_matches_np_convolve_with_reversed_taps():
    rng = np.random.default_rng(7)
    W, C, L = 4, 6, 25
    w = rng.uniform(-0.5, 0.5, (C, W))
    b = rng.uniform(-0.5, 0.5, C)
    win0 = rng.standard_normal((W - 1, C))
    u = rng.standard_normal((L, C))
    v = orc.conv_tokens(win0, u, w, b)
    stream = np.concatenate([win0, u])
    for c in range(C):
        ref = np.convolve(stream[:, c], w[c, ::-1], mode="valid") + b[c]
        assert np.allclose(v[:, c], ref, rtol=1e-14, atol=1e-14)


def test_decode_conv_window_is_exact_copy_and_matches_np_convolve():
    rng = np.random.default_rng(8)
    shape = synth.TINY
    params, ssm0, conv0, u, z, dt = synth.random_problem(rng, shape, 5)
    pool = orc.PoolRef(shape, 1, 2, "f64", "f64")
    pool.ssm[0, 1], pool.conv[0, 1] = ssm0, conv0
    stream = np.concatenate([conv0.T, u])
    for t in range(5):
        orc.decode_step(pool, 0, params, [1], u[t:t + 1], z[t:t + 1], dt[t:t + 1], "f64")
        assert np.array_equal(pool.conv[0, 1], stream[t + 1:t + 4].T)
    # the decode conv value (through x of head 0 after one step) against np.convolve
    pool2 = orc.PoolRef(shape, 1, 1, "f64", "f64")
    pool2.conv[0, 0] = conv0
    D0 = dict(params, D=np.ones(shape.nheads))
    zbig = np.full((1, shape.intermediate), 50.0)          # SiLU(50) = 50 to 1e-20
    out = orc.decode_step(pool2, 0, D0, [0], u[:1], zbig, np.full((1, shape.nheads), -80.0), "f64")
    # with Delta ~ e^-84 the state term vanishes: out = (C.h0*alpha + x) * 50 with h0 = 0
    c = 3
    ref_v = np.convolve(stream[:4, c], params["conv_w"][c, ::-1], mode="valid")[0] + params["conv_b"][c]
    assert math.isclose(out[0, c] / 50.0, ref_v * scipy.special.expit(ref_v), rel_tol=1e-12)


# ---------------------------------------------------------------- recurrence
def _post_conv(params, shape, conv0, u, dt):
    act = orc.silu(orc.conv_tokens(conv0.T, u, params["conv_w"], params["conv_b"]))
    I, G, N = shape.intermediate, shape.n_groups, shape.d_state
    x = act[:, :I].reshape(len(u), shape.nheads, shape.head_dim)
    B = act[:, I:I + G * N].reshape(len(u), G, N)
    C = act[:, I + G * N:].reshape(len(u), G, N)
    delta = np.logaddexp(0.0, dt + params["dt_bias"])
    return x, B, C, delta


@pytest.mark.parametrize("shape,L,seed", [
    (synth.TINY, 24, 0),
    (synth.Shape(4, 8, 8, 2, 4), 40, 1),
    (synth.Shape(6, 4, 5, 3, 3), 17, 2),
    (synth.Shape(2, 3, 7, 1, 2), 1, 3),
])
def test_prefill_equals_semiseparable_matrix_form(shape, L, seed):
    rng = np.random.default_rng(seed)
    params, ssm0, conv0, u, z, dt = synth.random_problem(rng, shape, L)
    pool = orc.PoolRef(shape, 1, 3, "f64", "f64")
    pool.ssm[0, 2], pool.conv[0, 2] = ssm0, conv0
    out = orc.prefill(pool, 0, params, [0, L], [2], [1], [0], u, z, dt, "f64")
    x, B, C, delta = _post_conv(params, shape, conv0, u, dt)
    hpg = shape.nheads // shape.n_groups
    P = shape.head_dim
    for h in range(shape.nheads):
        g = h // hpg
        Y = orc.ssd_matrix_form(ssm0[h], x[:, h], B[:, g], C[:, g], delta[:, h],
                                params["A"][h], params["D"][h])
        gate = z[:, h * P:(h + 1) * P] * scipy.special.expit(z[:, h * P:(h + 1) * P])
        assert rel_err(out[:, h * P:(h + 1) * P], Y * gate) < 1e-12


@pytest.mark.parametrize("L", [1, 16, 40])
def test_ssm_scan_equals_matrix_form(L):
    rng = np.random.default_rng(100 + L)
    P, N = 3, 5
    x, B, C = rng.standard_normal((L, P)), rng.standard_normal((L, N)), rng.standard_normal((L, N))
    delta = np.logaddexp(0.0, rng.standard_normal(L) - 3.0)
    A, D = -np.exp(rng.uniform(0, math.log(16))), rng.standard_normal()
    h0 = rng.normal(0, 0.1, (P, N))
    y, _ = orc.ssm_scan(h0, x, B, C, delta, A, D)
    assert rel_err(y, orc.ssd_matrix_form(h0, x, B, C, delta, A, D)) < 1e-12


def test_constant_input_closed_form():
    """u_t = u with the initial window = u, and constant z, dt: a geometric series."""
    shape = synth.Shape(4, 8, 6, 2, 4)
    rng = np.random.default_rng(11)
    params = synth.layer_params(rng, shape)
    L = 40
    u1 = rng.standard_normal(shape.conv_dim)
    z1 = rng.standard_normal(shape.intermediate)
    dt1 = rng.standard_normal(shape.nheads)
    h0 = rng.normal(0, 0.1, (shape.nheads, shape.head_dim, shape.d_state))
    pool = orc.PoolRef(shape, 1, 1, "f64", "f64")
    pool.ssm[0, 0] = h0
    pool.conv[0, 0] = np.repeat(u1[:, None], shape.conv_kernel - 1, axis=1)
    u, z, dt = np.tile(u1, (L, 1)), np.tile(z1, (L, 1)), np.tile(dt1, (L, 1))
    out = orc.prefill(pool, 0, params, [0, L], [0], [1], [0], u, z, dt, "f64")
    # closed form
    v = params["conv_b"] + u1 * params["conv_w"].sum(axis=1)
    act = v * scipy.special.expit(v)
    I, G, N, P, H = shape.intermediate, shape.n_groups, shape.d_state, shape.head_dim, shape.nheads
    x = act[:I].reshape(H, P)
    B = act[I:I + G * N].reshape(G, N)
    C = act[I + G * N:].reshape(G, N)
    delta = np.logaddexp(0.0, dt1 + params["dt_bias"])
    alpha = np.exp(delta * params["A"])
    g = np.arange(H) // (H // G)
    inject = (delta[:, None] * x)[:, :, None] * B[g][:, None, :]
    gate = z1 * scipy.special.expit(z1)
    for t in (0, 1, 9, L - 1):
        n = t + 1
        h = alpha[:, None, None] ** n * h0 + ((1 - alpha ** n) / (1 - alpha))[:, None, None] * inject
        y = np.einsum("hpn,hn->hp", h, C[g]) + params["D"][:, None] * x
        assert rel_err(out[t], y.reshape(-1) * gate) < 1e-12
    assert rel_err(pool.ssm[0, 0], h) < 1e-12


def test_scalar_case_is_an_iir_filter():
    """H = P = N = G = 1 with constant Delta: h is lfilter([1], [1, -alpha], Delta x B, zi = alpha h0)."""
    shape = synth.Shape(1, 1, 1, 1, 4)
    rng = np.random.default_rng(5)
    params = synth.layer_params(rng, shape)
    L = 64
    u = rng.standard_normal((L, shape.conv_dim))
    z = np.full((L, 1), 40.0)                    # gate ~ 40 exactly enough; compared after division
    dt = np.full((L, 1), 0.3)
    h0 = np.array([[[0.25]]])
    pool = orc.PoolRef(shape, 1, 1, "f64", "f64")
    pool.ssm[0, 0] = h0
    conv0 = rng.standard_normal((shape.conv_dim, 3))
    pool.conv[0, 0] = conv0
    # make the readout the state itself: D = 0 and read C through the closed conv
    p2 = dict(params, D=np.zeros(1))
    out = orc.prefill(pool, 0, p2, [0, L], [0], [1], [0], u, z, dt, "f64")
    x, B, C, delta = _post_conv(p2, shape, conv0, u, dt)
    alpha = math.exp(delta[0, 0] * p2["A"][0])
    drive = delta[:, 0] * x[:, 0, 0] * B[:, 0, 0]
    h, _ = scipy.signal.lfilter([1.0], [1.0, -alpha], drive, zi=[alpha * h0[0, 0, 0]])
    y_ref = h * C[:, 0, 0] * (z[:, 0] * scipy.special.expit(z[:, 0]))
    assert rel_err(out[:, 0], y_ref) < 1e-12
    assert math.isclose(pool.ssm[0, 0, 0, 0, 0], h[-1], rel_tol=1e-12)


# ---------------------------------------------------------------- page snippet
def test_affine_composition_and_restored_error_from_the_page(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "affine_snippet.json")))
    steps = g["steps"]
    # realise step (a_t, b_t) as alpha_t = exp(Delta_t A) with A = -1, and Delta_t x_t B_t = b_t
    delta = np.array([-math.log(a) for a, _ in steps])
    x = np.array([[b / d] for (_, b), d in zip(steps, delta)])
    Bm, Cm = np.ones((3, 1)), np.ones((3, 1))
    _, b_comp = orc.ssm_scan(np.zeros((1, 1)), x, Bm, Cm, delta, -1.0, 0.0)
    _, a_comp = orc.ssm_scan(np.ones((1, 1)), np.zeros((3, 1)), Bm, Cm, delta, -1.0, 0.0)
    assert math.isclose(a_comp[0, 0], g["composed_by_hand"]["a"], rel_tol=1e-12)
    assert math.isclose(b_comp[0, 0], g["composed_by_hand"]["b"], rel_tol=1e-12)
    r = g["restored_error"]
    n = r["steps"]
    for factor in r["factors"]:
        d = np.ones(n)
        xin = np.full((n, 1), r["input"])
        _, h_exact = orc.ssm_scan(np.full((1, 1), r["exact_start"]), xin, np.ones((n, 1)),
                                  np.ones((n, 1)), d, math.log(factor), 0.0)
        _, h_rest = orc.ssm_scan(np.full((1, 1), r["restored_start"]), xin, np.ones((n, 1)),
                                 np.ones((n, 1)), d, math.log(factor), 0.0)
        assert np.isclose(h_rest[0, 0] - h_exact[0, 0], 0.01 * factor ** n)


def test_linearity_in_initial_state():
    shape = synth.Shape(4, 8, 8, 2, 4)
    rng = np.random.default_rng(21)
    params, ssm0, conv0, u, z, dt = synth.random_problem(rng, shape, 30)
    dlt = rng.normal(0, 0.01, ssm0.shape)
    outs, states = [], []
    for h0 in (ssm0, ssm0 + dlt):
        pool = orc.PoolRef(shape, 1, 1, "f64", "f64")
        pool.ssm[0, 0], pool.conv[0, 0] = h0, conv0
        outs.append(orc.prefill(pool, 0, params, [0, 30], [0], [1], [0], u, z, dt, "f64"))
        states.append(pool.ssm[0, 0].copy())
    delta = np.logaddexp(0.0, dt + params["dt_bias"])
    decay = np.exp((delta * params["A"]).sum(axis=0))     # prod_t alpha_t per head
    assert rel_err(states[1] - states[0], decay[:, None, None] * dlt) < 1e-9


# ---------------------------------------------------------------- invariants
def _fresh(shape, slots, dtype="f64"):
    return orc.PoolRef(shape, 1, slots, dtype, dtype)


def test_prefill_handoff_equals_one_call():
    shape = synth.TINY
    rng = np.random.default_rng(31)
    params, ssm0, conv0, u, z, dt = synth.random_problem(rng, shape, 50)
    one = _fresh(shape, 1)
    one.ssm[0, 0], one.conv[0, 0] = ssm0, conv0
    y1 = orc.prefill(one, 0, params, [0, 50], [0], [1], [0], u, z, dt, "f64")
    two = _fresh(shape, 1)
    two.ssm[0, 0], two.conv[0, 0] = ssm0, conv0
    ya = orc.prefill(two, 0, params, [0, 16], [0], [1], [0], u[:16], z[:16], dt[:16], "f64")
    yb = orc.prefill(two, 0, params, [0, 34], [0], [1], [16], u[16:], z[16:], dt[16:], "f64")
    assert rel_err(np.concatenate([ya, yb]), y1) < 1e-12
    assert rel_err(two.ssm[0, 0], one.ssm[0, 0]) < 1e-12
    assert np.array_equal(two.conv[0, 0], one.conv[0, 0])


@pytest.mark.parametrize("dtype,tol", [("f64", 1e-12), ("f32", 2e-6)])
def test_decode_steps_equal_prefill(dtype, tol):
    shape = synth.TINY
    rng = np.random.default_rng(41)
    params, ssm0, conv0, u, z, dt = synth.random_problem(rng, shape, 20)
    dec = _fresh(shape, 1, dtype)
    dec.ssm[0, 0], dec.conv[0, 0] = ssm0, conv0
    ys = [orc.decode_step(dec, 0, params, [0], u[t:t + 1], z[t:t + 1], dt[t:t + 1], dtype)[0]
          for t in range(20)]
    pre = _fresh(shape, 1, dtype)
    pre.ssm[0, 0], pre.conv[0, 0] = ssm0, conv0
    yp = orc.prefill(pre, 0, params, [0, 20], [0], [1], [0], u, z, dt, dtype)
    assert rel_err(np.array(ys), yp) < tol
    assert rel_err(dec.ssm[0, 0], pre.ssm[0, 0]) < tol
    assert np.array_equal(dec.conv[0, 0], pre.conv[0, 0])


def test_checkpoints_equal_prefix_prefills():
    shape = synth.TINY
    rng = np.random.default_rng(51)
    params, ssm0, conv0, u, z, dt = synth.random_problem(rng, shape, 30)
    pool = _fresh(shape, 6, "f32")
    pool.ssm[0, 0], pool.conv[0, 0] = ssm0, conv0
    ck = np.array([[3, 5, 4]])
    orc.prefill(pool, 0, params, [0, 30], [0], [1], [0], u, z, dt, "f32", ckpt_interval=8, ckpt_slots=ck)
    for k, p in enumerate((8, 16, 24)):
        ref = _fresh(shape, 1, "f32")
        ref.ssm[0, 0], ref.conv[0, 0] = ssm0, conv0
        orc.prefill(ref, 0, params, [0, p], [0], [1], [0], u[:p], z[:p], dt[:p], "f32")
        assert np.array_equal(pool.ssm[0, ck[0, k]], ref.ssm[0, 0])
        assert np.array_equal(pool.conv[0, ck[0, k]], ref.conv[0, 0])
    # start_pos shifts the checkpoint grid to absolute positions
    pool2 = _fresh(shape, 6, "f32")
    pool2.ssm[0, 0], pool2.conv[0, 0] = ssm0, conv0
    orc.prefill(pool2, 0, params, [0, 30], [0], [1], [4], u, z, dt, "f32", ckpt_interval=8,
                ckpt_slots=np.array([[1, 2, 3, 4]]))
    ref = _fresh(shape, 1, "f32")
    ref.ssm[0, 0], ref.conv[0, 0] = ssm0, conv0
    orc.prefill(ref, 0, params, [0, 4], [0], [1], [4], u[:4], z[:4], dt[:4], "f32")
    assert np.array_equal(pool2.ssm[0, 1], ref.ssm[0, 0])      # absolute position 8


@pytest.mark.parametrize("shape,heads", [
    (synth.Shape(6, 4, 8, 3, 4), [5, 0, 3]),         # three groups of two heads, one head of each, unsorted
    (synth.Shape(8, 8, 16, 2, 3), [7, 1, 2]),        # two groups of four heads
    (synth.Shape(4, 8, 8, 2, 2), [2]),               # a single head of the second group
])
def test_head_subset_prefill_equals_full_prefill(shape, heads):
    """prefill(heads=...) runs the recurrence of the chosen heads only; their output columns,
    final states and checkpoint states equal those of the full-head call, heads of other groups
    included (the group map, the x, B, C channel selection and the z columns), and nothing else
    of the states is written."""
    rng = np.random.default_rng(71)
    lens = [13, 1, 22]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T = int(cu[-1])
    params, _, _, u, z, dt = synth.random_problem(rng, shape, T)
    slots, has_init, start = [1, 4, 6], [1, 0, 1], [5, 0, 8]
    ck = np.array([[2, 3, -1], [-1, -1, -1], [5, 7, 0]])
    nslot = 10

    def run(heads_arg):
        pool = _fresh(shape, nslot, "f32")
        r = np.random.default_rng(72)
        pool.ssm[0] = r.standard_normal(pool.ssm[0].shape)
        pool.conv[0] = r.standard_normal(pool.conv[0].shape)
        before = pool.ssm.copy()
        y = orc.prefill(pool, 0, params, cu, slots, has_init, start, u, z, dt, "f64", ckpt_interval=4,
                        ckpt_slots=ck, heads=heads_arg)
        return pool, before, y

    full, _, y_full = run(None)
    sub, before, y_sub = run(heads)
    H, P = shape.nheads, shape.head_dim
    other = [h for h in range(H) if h not in heads]
    ys, yf = y_sub.reshape(T, H, P), y_full.reshape(T, H, P)
    assert rel_err(ys[:, heads], yf[:, heads]) <= 1e-12
    assert np.all(np.isnan(ys[:, other]))
    written = set(slots) | {int(c) for c in ck.ravel() if c >= 0}
    assert len(written) == 8                     # three finals and five checkpoints, all distinct
    for s in written:
        assert rel_err(sub.ssm[0, s][heads], full.ssm[0, s][heads]) <= 1e-12
        assert np.array_equal(sub.ssm[0, s][other], before[0, s][other])    # other heads untouched
        assert np.array_equal(sub.conv[0, s], full.conv[0, s])              # windows in full
    for s in set(range(nslot)) - written:
        assert np.array_equal(sub.ssm[0, s], before[0, s])


def test_padding_rows_and_fresh_sequences_do_not_read_slots():
    shape = synth.TINY
    rng = np.random.default_rng(61)
    params, ssm0, conv0, u, z, dt = synth.random_problem(rng, shape, 4)
    pool = _fresh(shape, 4, "f32")
    pool.ssm[:] = np.nan
    pool.conv[:] = np.nan
    pool.ssm[0, 2], pool.conv[0, 2] = ssm0, conv0
    y = orc.decode_step(pool, 0, params, [-1, 2], u[:2], z[:2], dt[:2], "f32")
    assert np.all(y[0] == 0) and np.all(np.isfinite(y[1]))
    for s in (0, 1, 3):
        assert np.all(np.isnan(pool.ssm[0, s])) and np.all(np.isnan(pool.conv[0, s]))
    y2 = orc.prefill(pool, 0, params, [0, 4], [1], [0], [0], u, z, dt, "f32")
    assert np.all(np.isfinite(y2)) and np.all(np.isfinite(pool.ssm[0, 1]))


# ---------------------------------------------------------------- byte counts
def test_state_bytes_match_the_pages(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "state_sizes.json")))
    shape = synth.NEMOTRON_H
    by = {e["id"]: e for e in g["entries"]}

    def per_layer(ssm, conv):
        p = orc.PoolRef(shape, 1, 1, ssm, conv or "bf16")
        return p.ssm_bytes_per_slot_layer() + (p.conv_bytes_per_slot_layer() if conv else 0)

    e = by["bf16_ssm_per_layer"]
    assert per_layer("bf16", None) == 2 * 2 ** 20
    assert e["layers"] * per_layer("bf16", None) == e["total_bytes"] == e["mib"] * 2 ** 20
    e = by["fp32_ssm_bf16_conv_24_layers"]
    total = e["layers"] * per_layer("f32", "bf16")
    assert total == e["total_bytes"]
    assert int(total // e["kv_bytes_per_token"]) == e["crossover_tokens"]
    e = by["bf16_ssm_bf16_conv_24_layers"]
    assert int(e["layers"] * per_layer("bf16", "bf16") // e["kv_bytes_per_token"]) == e["crossover_tokens"]
    e = by["per_layer_block_mib"]
    assert round(per_layer("f32", "bf16") / 2 ** 20, 2) == e["mib_2dp"]
    e = by["pool_256_slots_gib"]
    assert round(e["slots"] * e["layers"] * per_layer("f32", "bf16") / 2 ** 30, 1) == e["gib_1dp"]
    e = by["conv_share_percent"]
    p = orc.PoolRef(shape, 1, 1, "f32", "bf16")
    assert round(100 * p.conv_bytes_per_slot_layer() / per_layer("f32", "bf16"), 1) == e["percent_1dp"]
    e = by["long_context_per_layer"]
    assert e["seqs"] * per_layer("f32", None) == e["total_bytes"]


# ---------------------------------------------------------------- pin strength
def test_pins_catch_planted_mistakes():
    """Mistakes planted in a copy of the scan are caught by the matrix-form pin."""
    rng = np.random.default_rng(71)
    L, P, N = 12, 3, 4
    x, B, C = rng.standard_normal((L, P)), rng.standard_normal((L, N)), rng.standard_normal((L, N))
    delta = np.logaddexp(0.0, rng.standard_normal(L) - 2.0)
    A, D = -2.0, 0.7
    h0 = rng.normal(0, 0.1, (P, N))
    ref = orc.ssd_matrix_form(h0, x, B, C, delta, A, D)

    def scan(variant):
        h = h0.copy()
        y = np.zeros((L, P))
        for t in range(L):
            h_old = h
            if variant == "no_delta_on_input":
                h = np.exp(delta[t] * A) * h + np.outer(x[t], B[t])
            elif variant == "sign_of_A":
                h = np.exp(-delta[t] * A) * h + delta[t] * np.outer(x[t], B[t])
            elif variant == "readout_old_state":
                h = np.exp(delta[t] * A) * h + delta[t] * np.outer(x[t], B[t])
                y[t] = h_old @ C[t] + D * x[t]
                continue
            elif variant == "B_C_swapped":
                h = np.exp(delta[t] * A) * h + delta[t] * np.outer(x[t], C[t])
                y[t] = h @ B[t] + D * x[t]
                continue
            elif variant == "no_D":
                h = np.exp(delta[t] * A) * h + delta[t] * np.outer(x[t], B[t])
                y[t] = h @ C[t]
                continue
            elif variant == "input_index_shift":
                h = np.exp(delta[t] * A) * h + delta[t] * np.outer(x[t - 1], B[t])
            y[t] = h @ C[t] + D * x[t]
        return y

    for v in ("no_delta_on_input", "sign_of_A", "readout_old_state", "B_C_swapped", "no_D",
              "input_index_shift"):
        assert rel_err(scan(v), ref) > 1e-3, v
    assert rel_err(orc.ssm_scan(h0, x, B, C, delta, A, D)[0], ref) < 1e-12


# ---------------------------------------------------------------- int8 checkpoint store
def test_int8_codes_of_exact_multiples_and_reduction_axis():
    """States built as code * 2^-k with a different k per (head, d_state index) and a +-127 in
    every such column: quantizing returns those codes and scales 2^-k exactly (so one scale per
    (head, n), taken over head_dim), and dequantizing returns the state exactly."""
    rng = np.random.default_rng(41)
    H, P, N = 3, 8, 5
    codes = rng.integers(-127, 128, (H, P, N))
    rows = rng.integers(0, P, (H, N))
    sign = rng.choice([-1, 1], (H, N))
    for h in range(H):
        for n in range(N):
            codes[h, rows[h, n], n] = 127 * sign[h, n]
    k = rng.integers(3, 12, (H, N))
    state = codes * np.exp2(-k.astype(np.float64))[:, None, :]
    q, s = orc.int8_quantize(state)
    assert q.dtype == np.int8 and s.shape == (H, N)
    assert np.array_equal(q.astype(np.int64), codes)
    assert np.array_equal(s.astype(np.float64), np.exp2(-k.astype(np.float64)))
    assert np.array_equal(orc.int8_dequantize(q, s, "f32"), state)
    assert np.array_equal(orc.int8_quantize(-state)[0].astype(np.int64), -codes)


def test_int8_codes_round_half_to_even():
    """amax = 127/128 makes the multiplier exactly 128: halves land on the even code."""
    vals = np.array([127.0, 2.5, 3.5, -2.5, 0.5, 1.5, -0.5, 126.5]) / 128.0
    q, s = orc.int8_quantize(vals.reshape(1, -1, 1))
    assert q[0, :, 0].tolist() == [127, 2, 4, -2, 0, 2, 0, 126]
    assert s[0, 0] == np.float32(1.0 / 128.0)


def test_int8_zero_column_and_error_bound():
    rng = np.random.default_rng(42)
    state = orc.round_to(rng.normal(0, 0.1, (4, 16, 32)), "bf16")
    state[1, :, 7] = 0.0
    q, s = orc.int8_quantize(state)
    assert s[1, 7] == 0 and not q[1, :, 7].any()
    restored = orc.int8_dequantize(q, s, "f32")
    amax = np.max(np.abs(state), axis=1)                    # per (head, n), in fp64
    # half a quantization step, plus the fp32 roundings of the multiplier and of the product
    bound = amax / 254.0 * (1 + 2.0 ** -20) + np.abs(state).max() * 2.0 ** -22
    assert np.all(np.abs(restored - state) <= bound[:, None, :])
    assert np.all(np.max(np.abs(q.astype(np.int64)), axis=1)[amax > 0] == 127)


def test_int8_store_holds_about_twice_the_cached_states_of_bf16():
    """[SSM-hybrids], SGLang int8 checkpoint passage: about twice as many cached states as bf16.
    At the Nemotron-H layer shape the int8 codes are half the bf16 state; with the per-(head, n)
    scales and the bf16 conv window kept native, an entry is 1.84x smaller than a bf16 slot."""
    sh = synth.NEMOTRON_H
    pool = orc.PoolRef(sh, 1, 1, "bf16", "bf16")
    st = orc.Int8StoreRef(pool, 1)
    entry = st.codes.nbytes + st.scales.nbytes + st.conv.size * 2
    slot = pool.ssm_bytes_per_slot_layer() + pool.conv_bytes_per_slot_layer()
    assert 2 * st.codes.nbytes == pool.ssm_bytes_per_slot_layer()
    assert 1.8 < slot / entry < 2.0


def test_int8_restored_error_evolves_through_the_decay_product():
    """[SSM-hybrids], the affine-composition passage: an error in a restored state evolves through
    the product of the later transition factors.  Restoring an int8 entry and continuing with the
    same inputs leaves the state off by (prod_t alpha_t) times the quantization error."""
    shape = synth.Shape(4, 8, 16, 2, 4)
    rng = np.random.default_rng(43)
    params, ssm0, conv0, u, z, dt = synth.random_problem(rng, shape, 40)
    ssm0 = orc.round_to(ssm0, "bf16")
    pool = orc.PoolRef(shape, 1, 3, "bf16", "bf16")
    pool.ssm[0, 0], pool.conv[0, 0] = ssm0, orc.round_to(conv0, "bf16")
    store = orc.Int8StoreRef(pool, 2)
    orc.int8_store_put(pool, store, 0, [0], [1])
    orc.int8_store_get(store, pool, 0, [1], [2])
    assert np.array_equal(pool.conv[0, 2], pool.conv[0, 0])
    err0 = pool.ssm[0, 2] - pool.ssm[0, 0]
    assert 0 < np.abs(err0).max() <= np.abs(ssm0).max() / 127
    finals = []
    for slot in (0, 2):
        run = orc.PoolRef(shape, 1, 1, "f64", "f64")
        run.ssm[0, 0], run.conv[0, 0] = pool.ssm[0, slot], pool.conv[0, slot]
        orc.prefill(run, 0, params, [0, 40], [0], [1], [0], u, z, dt, "f64")
        finals.append(run.ssm[0, 0].copy())
    delta = np.logaddexp(0.0, dt + params["dt_bias"])
    decay = np.exp((delta * params["A"]).sum(axis=0))
    assert rel_err(finals[1] - finals[0], decay[:, None, None] * err0) < 1e-9


# ---------------------------------------------------------------- multi-token (speculative) decode
def test_multi_token_decode_snapshots_equal_prefill_checkpoints_at_every_token():
    """K decode tokens with a snapshot after each equal, with fp32 state, a prefill of the same
    tokens that checkpoints after every token (the prefill keeps the state unrounded between
    tokens; the difference is fp32 rounding), and the outputs match the prefill's."""
    shape = synth.Shape(4, 8, 16, 2, 4)
    rng = np.random.default_rng(51)
    K = 5
    params, ssm0, conv0, u, z, dt = synth.random_problem(rng, shape, K)
    a = orc.PoolRef(shape, 1, 8, "f32", "f32")
    a.ssm[0, 0], a.conv[0, 0] = ssm0, conv0
    y_multi = orc.decode_multi(a, 0, params, [0], [[1, 2, 3, 4, 5]], u[None], z[None], dt[None], "f64")
    b = orc.PoolRef(shape, 1, 8, "f32", "f32")
    b.ssm[0, 0], b.conv[0, 0] = ssm0, conv0
    y_pre = orc.prefill(b, 0, params, [0, K], [0], [1], [0], u, z, dt, "f64", ckpt_interval=1,
                        ckpt_slots=[[1, 2, 3, 4, 5]])
    assert rel_err(y_multi[0], y_pre) < 1e-6
    for t in range(K):
        assert rel_err(a.ssm[0, 1 + t], b.ssm[0, 1 + t]) < 1e-6
        assert np.array_equal(a.conv[0, 1 + t], b.conv[0, 1 + t])
    assert np.array_equal(a.ssm[0, 0], orc.round_to(ssm0, "f32"))     # the input slot is left as it was


def test_multi_token_decode_pads_and_skips():
    shape = synth.TINY
    rng = np.random.default_rng(52)
    params, ssm0, conv0, u, z, dt = synth.random_problem(rng, shape, 3)
    pool = orc.PoolRef(shape, 1, 4, "f32", "f32")
    pool.ssm[0, 2], pool.conv[0, 2] = ssm0, conv0
    uu = np.stack([u, u]); zz = np.stack([z, z]); dd = np.stack([dt, dt])
    y = orc.decode_multi(pool, 0, params, [-1, 2], [[0, 1, 3], [-1, 3, -1]], uu, zz, dd, "f32")
    assert not y[0].any() and y[1].any()
    assert not pool.ssm[0, 0].any() and not pool.ssm[0, 1].any()      # the padding row wrote nothing
    ref = orc.PoolRef(shape, 1, 1, "f32", "f32")
    ref.ssm[0, 0], ref.conv[0, 0] = ssm0, conv0
    for t in range(2):
        orc.decode_step(ref, 0, params, [0], u[t:t + 1], z[t:t + 1], dt[t:t + 1], "f32")
    assert np.array_equal(pool.ssm[0, 3], ref.ssm[0, 0])               # the state after token 1


# ---------------------------------------------------------------- Mamba1 decode (second family)
def _m1_params(rng, D, N, W=4):
    return dict(A=-np.exp(rng.uniform(0.0, 2.0, (D, N))), D=rng.normal(0, 1, D), dt_bias=rng.uniform(-4, -2, D),
                conv_w=rng.uniform(-0.5, 0.5, (D, W)), conv_b=rng.uniform(-0.5, 0.5, D))


def test_mamba1_with_one_decay_per_channel_equals_mamba2_with_one_channel_heads():
    """With A[d, n] = a_d for every n, Mamba1 over D channels is Mamba2 with D heads of head_dim 1
    and one group, given the same post-conv B and C: the Mamba2 side gets B and C through a conv
    with taps (0, .., 0, 1) and no bias, fed the SiLU preimages of the wanted values."""
    import scipy.optimize
    rng = np.random.default_rng(61)
    D, N, W, steps = 6, 8, 4, 5
    p1 = _m1_params(rng, D, N, W)
    a = -np.exp(rng.uniform(0, 2, D))
    p1["A"] = np.repeat(a[:, None], N, axis=1)
    sh2 = synth.Shape(D, 1, N, 1, W)
    Cd = sh2.conv_dim                                   # D + 2N channels: [x | B | C]
    p2 = dict(A=a, D=p1["D"], dt_bias=p1["dt_bias"], conv_w=np.zeros((Cd, W)), conv_b=np.zeros(Cd))
    p2["conv_w"][:D], p2["conv_b"][:D] = p1["conv_w"], p1["conv_b"]
    p2["conv_w"][D:, W - 1] = 1.0
    silu_inv = lambda t: scipy.optimize.brentq(lambda v: v / (1 + math.exp(-v)) - t, -1.0, 50.0, xtol=1e-15)
    m1 = orc.Mamba1PoolRef(D, N, W, 1, 1, "f64", "f64")
    m2 = orc.PoolRef(sh2, 1, 1, "f64", "f64")
    h0 = rng.normal(0, 0.1, (D, N))
    win = rng.normal(0, 0.1, (D, W - 1))
    m1.ssm[0, 0], m1.conv[0, 0] = h0, win
    m2.ssm[0, 0] = h0[:, None, :]
    m2.conv[0, 0][:D] = win
    for t in range(steps):
        u = rng.normal(0, 1, D)
        z = rng.normal(0, 1, D)
        dt = rng.normal(0, 1, D)
        Bt, Ct = rng.uniform(0.1, 2.0, N), rng.uniform(0.1, 2.0, N)
        y1 = orc.mamba1_decode_step(m1, 0, p1, [0], u[None], z[None], dt[None], Bt[None], Ct[None], "f64")
        u2 = np.concatenate([u, [silu_inv(v) for v in Bt], [silu_inv(v) for v in Ct]])
        y2 = orc.decode_step(m2, 0, p2, [0], u2[None], z[None], dt[None], "f64")
        assert rel_err(y1, y2) < 1e-11, t
        assert rel_err(m1.ssm[0, 0], m2.ssm[0, 0][:, 0, :]) < 1e-11, t
        assert np.array_equal(m1.conv[0, 0], m2.conv[0, 0][:D])


def test_mamba1_constant_input_closed_form_per_channel_and_state_index():
    """Constant inputs: every (d, n) follows its own geometric series with ratio exp(Delta_d A[d, n])."""
    rng = np.random.default_rng(62)
    D, N, W, T = 4, 6, 4, 9
    p = _m1_params(rng, D, N, W)
    u = rng.normal(0, 1, D)
    pool = orc.Mamba1PoolRef(D, N, W, 1, 1, "f64", "f64")
    h0 = rng.normal(0, 0.1, (D, N))
    pool.ssm[0, 0], pool.conv[0, 0] = h0, np.repeat(u[:, None], W - 1, axis=1)   # window already = u
    z, dt = rng.normal(0, 1, D), rng.normal(0, 1, D)
    Bt, Ct = rng.normal(0, 1, N), rng.normal(0, 1, N)
    for _ in range(T):
        y = orc.mamba1_decode_step(pool, 0, p, [0], u[None], z[None], dt[None], Bt[None], Ct[None], "f64")
    x = u * 0 + (p["conv_b"] + p["conv_w"].sum(axis=1) * u)
    x = x / (1 + np.exp(-x))
    delta = np.log1p(np.exp(dt + p["dt_bias"]))
    al = np.exp(delta[:, None] * p["A"])
    inj = (delta * x)[:, None] * Bt[None, :]
    hT = al ** T * h0 + (1 - al ** T) / (1 - al) * inj
    assert rel_err(pool.ssm[0, 0], hT) < 1e-12
    yT = (hT @ Ct + p["D"] * x) * (z / (1 + np.exp(-z)))
    assert rel_err(y[0], yT) < 1e-12


def test_mamba1_prefill_equals_decode_steps_and_the_decay_product():
    """A Mamba1 prefill equals the same tokens as decode steps (fp64 storage: no rounding between
    tokens either way), checkpoints included, and a perturbation of the initial state evolves
    through the product of the decays exp(sum_t Delta_t[d] A[d, n])."""
    rng = np.random.default_rng(63)
    D, N, W, L = 8, 8, 3, 21
    p = _m1_params(rng, D, N, W)
    u, z, dt = rng.normal(0, 1, (L, D)), rng.normal(0, 1, (L, D)), rng.normal(0, 1, (L, D))
    Bm, Cm = rng.normal(0, 1, (L, N)), rng.normal(0, 1, (L, N))
    h0, w0 = rng.normal(0, 0.1, (D, N)), rng.normal(0, 0.1, (D, W - 1))
    pre = orc.Mamba1PoolRef(D, N, W, 1, 6, "f64", "f64")
    pre.ssm[0, 1], pre.conv[0, 1] = h0, w0
    y_pre = orc.mamba1_prefill(pre, 0, p, [0, L], [1], [1], [3], u, z, dt, Bm, Cm, "f64", ckpt_interval=6,
                               ckpt_slots=[[2, 3, 4]])
    dec = orc.Mamba1PoolRef(D, N, W, 1, 1, "f64", "f64")
    dec.ssm[0, 0], dec.conv[0, 0] = h0, w0
    snaps = {}
    for t in range(L):
        y = orc.mamba1_decode_step(dec, 0, p, [0], u[t:t + 1], z[t:t + 1], dt[t:t + 1], Bm[t:t + 1], Cm[t:t + 1],
                                   "f64")
        assert rel_err(y[0], y_pre[t]) < 1e-12, t
        snaps[3 + t + 1] = (dec.ssm[0, 0].copy(), dec.conv[0, 0].copy())
    assert rel_err(pre.ssm[0, 1], dec.ssm[0, 0]) < 1e-12
    for k, pos in enumerate((6, 12, 18)):                       # multiples of 6 in (3, 24]
        assert rel_err(pre.ssm[0, 2 + k], snaps[pos][0]) < 1e-12
        assert np.array_equal(pre.conv[0, 2 + k], snaps[pos][1])
    dlt = rng.normal(0, 0.01, (D, N))
    pre2 = orc.Mamba1PoolRef(D, N, W, 1, 6, "f64", "f64")
    pre2.ssm[0, 1], pre2.conv[0, 1] = h0 + dlt, w0
    orc.mamba1_prefill(pre2, 0, p, [0, L], [1], [1], [3], u, z, dt, Bm, Cm, "f64")
    delta = np.logaddexp(0.0, dt + p["dt_bias"])                 # (L, D)
    decay = np.exp(delta.sum(axis=0)[:, None] * p["A"])         # prod_t exp(Delta_t[d] A[d, n])
    assert rel_err(pre2.ssm[0, 1] - pre.ssm[0, 1], decay * dlt) < 1e-9
