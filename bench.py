#!/usr/bin/env python3
"""Benchmark of the Mamba2 slot-pool hot path on one MI355X.

Step = one fused decode step of a Nemotron-H-shaped Mamba2 layer (H=128 heads
of P=64, N=128, G=8 groups, conv width 4) for 256 live sequences at randomly
permuted slots of a 512-slot bf16 pool: conv-window shift, conv + SiLU,
softplus, state update, readout, gate, in place on the pool.  Inputs are
synthetic (seeded, resident in HBM before timing).  A second leg times the
checkpoint copy (256 slot-to-slot copies of both state objects), which is also
the measured ceiling of a streaming kernel on the part, and the int8 checkpoint
store (256 slots quantized into entries and restored), and the multi-token
(speculative) decode of the same 256 sequences with 4 tokens each, and a Mamba1
decode step (the pool's second state family, D = 8192, N = 16).  A third
times the
chunked prefill of one 8192-token sequence (chunk 256) at the same shape; a
fourth the mixed continuous batch (32 prefills with checkpoints and 224
decodes on one stream) and the 2 x 131072-token long context through all 48
layer calls with fp32 state.

Prints one JSON line.  The decode step is timed after the memory-bound legs
(copies, int8 store, multi-token and Mamba1 legs), so that the GPU runs at its
steady clocks, and before the prefill legs.  `roofline.achieved` is the
algorithmic bytes of one decode launch divided by its average duration, timed
with HIP events on the stream the kernel runs on.  `cpu_baseline` is the fp64
CPU oracle on bounded samples of the decode step and of the two prefill
workloads, single-threaded, with the host's core count.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
HBM_PEAK_GBS = 8000.0         # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16


def decode_bytes_per_seq(sh, ssm_b=2, conv_b=2, io_b=2, y_b=2) -> int:
    """Algorithmic HBM bytes of one decode token: state and window read+write, u, z, dt in, y out."""
    state = 2 * sh.nheads * sh.head_dim * sh.d_state * ssm_b
    window = 2 * sh.conv_dim * (sh.conv_kernel - 1) * conv_b
    return state + window + (sh.conv_dim + sh.intermediate + sh.nheads) * io_b + sh.intermediate * y_b


def prefill_dense_flops_per_token(sh, Q) -> int:
    """MFMA flops of one prefill token, dense tiles: C.B^T per group, (M o L) X and the two state products per head."""
    return 2 * Q * sh.d_state * sh.n_groups + 2 * Q * sh.head_dim * sh.nheads + 4 * sh.nheads * sh.head_dim * sh.d_state


# Sources whose kernels the counter records describe; the copy kernel is in both because its
# counter readings scale the others'.  A record is reported only while these hash as recorded.
DECODE_SOURCES = ["recurrent_state_update_amd/csrc/decode.hip", "recurrent_state_update_amd/csrc/device_common.h",
                  "recurrent_state_update_amd/csrc/kernels.h", "recurrent_state_update_amd/csrc/ckpt.hip"]
PREFILL_SOURCES = ["recurrent_state_update_amd/csrc/prefill.hip", "recurrent_state_update_amd/csrc/prefill.h",
                   "recurrent_state_update_amd/csrc/device_common.h", "recurrent_state_update_amd/csrc/kernels.h",
                   "recurrent_state_update_amd/csrc/ckpt.hip"]
PREFILL_KERNELS = ["bc_kernel", "walk_kernel"]
COPY_PAIRS = 256      # slot pairs per timed checkpoint copy (the decode pool's 512 slots, halves swapped)


def source_sha(root: str, files) -> str:
    import hashlib
    return hashlib.sha256(b"".join(open(os.path.join(root, p), "rb").read() for p in files)).hexdigest()


def write_traffic_record(root: str, fetch_dir: str, write_dir: str) -> dict:
    """profiles/decode_traffic.json and profiles/prefill_traffic.json from the two counter runs of
    profiles/decode_256seq_hbm_traffic.md: average FETCH_SIZE and WRITE_SIZE (KiB) per dispatch of
    the decode kernel and of each kernel of the 8192-token prefill, each scaled by what the counter
    reads for the checkpoint copy of known size (COPY_PAIRS x (2 MiB of state + 60 KiB of conv
    window) per launch)."""
    import csv
    import glob

    def per_dispatch(d, part):
        # part: a substring of the kernel name, or a tuple of alternatives (mangled and demangled)
        parts = part if isinstance(part, tuple) else (part,)
        acc, names = {}, set()
        f = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)[0]
        for r in csv.DictReader(open(f)):
            if any(p in r["Kernel_Name"] for p in parts):
                acc[r["Dispatch_Id"]] = acc.get(r["Dispatch_Id"], 0.0) + float(r["Counter_Value"])
                names.add(r["Kernel_Name"])
        return list(acc.values()), sorted(names)

    avg = lambda v: sum(v) / len(v)
    known = COPY_PAIRS * (2097152 + 61440) / 1024           # KiB of state and conv window per copy launch
    cp_f = [v for v in per_dispatch(fetch_dir, "slot_copy_kernel")[0] if v > 10000]   # the timed copies
    cp_w = [v for v in per_dispatch(write_dir, "slot_copy_kernel")[0] if v > 10000]
    fs, ws = known / avg(cp_f), known / avg(cp_w)
    dec_name = ("_ZN2m213decode_kernel", "m2::decode_kernel<")   # not the Mamba1 or multi-token decode
    dec_f, dec_w = per_dispatch(fetch_dir, dec_name)[0], per_dispatch(write_dir, dec_name)[0]
    dec = {"kernel": "decode_kernel<bf16, N=128, W=4>", "workload": "decode step, 256 sequences, Nemotron-H layer shape",
           "source_sha256": source_sha(root, DECODE_SOURCES), "sources": DECODE_SOURCES,
           "fetch_kib_per_launch": avg(dec_f), "write_kib_per_launch": avg(dec_w), "fetch_scale": fs,
           "write_scale": ws, "traffic_bytes_per_launch": (avg(dec_f) * fs + avg(dec_w) * ws) * 1024}
    json.dump(dec, open(os.path.join(root, "profiles", "decode_traffic.json"), "w"), indent=1)
    kernels, total = [], 0.0
    for k in PREFILL_KERNELS:
        (f, names), (w, _) = per_dispatch(fetch_dir, k), per_dispatch(write_dir, k)
        b = (avg(f) * fs + avg(w) * ws) * 1024
        kernels.append({"kernel": names, "dispatches": len(f), "fetch_kib": avg(f), "write_kib": avg(w),
                        "read_bytes": avg(f) * fs * 1024, "write_bytes": avg(w) * ws * 1024})
        total += b
    pre = {"workload": "chunked prefill of one 8192-token sequence, chunk 256, Nemotron-H layer shape, bf16 state",
           "source_sha256": source_sha(root, PREFILL_SOURCES), "sources": PREFILL_SOURCES, "fetch_scale": fs,
           "write_scale": ws, "kernels": kernels, "traffic_bytes_per_call": total}
    json.dump(pre, open(os.path.join(root, "profiles", "prefill_traffic.json"), "w"), indent=1)
    return {"decode": dec, "prefill": pre}


def measured_traffic(root: str, record: str, sources, key: str):
    """HBM bytes from a committed counter record, if the kernel sources still hash as recorded."""
    try:
        rec = json.load(open(os.path.join(root, "profiles", record)))
        sha = source_sha(root, sources)
    except (OSError, ValueError, KeyError):
        return None
    return rec[key] if sha == rec.get("source_sha256") else None


def time_calls(fn, warm: int, reps: int, stream, e0, e1) -> float:
    """GPU milliseconds per call of fn over reps calls after warm untimed ones (at least one).
    The last untimed call is queued after the barrier, ahead of the first event, so the GPU is
    busy while the host enqueues the timed calls: the events then time the calls back to back,
    not the host's launch latency after the barrier."""
    import torch
    for _ in range(max(warm - 1, 0)):
        fn()
    torch.cuda.synchronize()
    fn()
    e0.record(stream)
    for _ in range(reps):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--cpu-seconds", type=float, default=6.0, help="budget of the decode part of the CPU-oracle baseline leg")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--write-traffic-record", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="write profiles/decode_traffic.json from the FETCH_SIZE and WRITE_SIZE counter runs and exit")
    ap.add_argument("--no-prefill-workloads", action="store_true",
                    help="skip the mixed-batch and long-context prefill timings")
    ap.add_argument("--no-int8-store", action="store_true", help="skip the int8 checkpoint-store timing")
    ap.add_argument("--no-multi-decode", action="store_true", help="skip the multi-token decode timing")
    ap.add_argument("--no-mamba1", action="store_true", help="skip the Mamba1 decode and prefill timings")
    ap.add_argument("--no-checkpoint-copy", action="store_true",
                    help="skip the checkpoint-copy timing (also the known-size copy that scales the byte counters)")
    args = ap.parse_args()
    if args.write_traffic_record:
        rec = write_traffic_record(ROOT, *args.write_traffic_record)
        print(json.dumps(rec))
        return 0
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (the decode step shards by "
              "sequence and needs no collective); run with --gpus 1", file=sys.stderr)
        return 2

    import torch
    from recurrent_state_update_amd import synth
    from recurrent_state_update_amd.pool import LayerWeights, Pool

    dev = "cuda"
    w = synth.decode_workload(1)
    sh, slots = w["shape"], w["slots"]
    batch = len(slots)
    pool = Pool.allocate(1, w["num_slots"], sh.nheads, sh.head_dim, sh.d_state, sh.n_groups, sh.conv_kernel,
                         torch.bfloat16, torch.bfloat16, dev)
    for i, s in enumerate(slots):
        pool.ssm[0, int(s)] = synth.to_torch(w["ssm0"][i], "bf16").to(dev)
        pool.conv[0, int(s)] = synth.to_torch(w["conv0"][i], "bf16").to(dev)
    W = LayerWeights.from_numpy(w["params"], dev)
    u = synth.to_torch(w["u"], "bf16").to(dev)
    z = synth.to_torch(w["z"], "bf16").to(dev)
    dt = synth.to_torch(w["dt"], "bf16").to(dev)
    x, B, C = pool.split_xbc(u)
    y = torch.empty((batch, sh.intermediate), dtype=torch.bfloat16, device=dev)
    sl = torch.from_numpy(slots).to(dev)
    pool.decode_step(0, W, sl, x, B, C, z, dt, y, slots_host=slots)   # validates once

    def step():
        pool.decode_step(0, W, sl, x, B, C, z, dt, y)

    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    legs = {}
    # The memory-bound legs run first: the GPU reaches its steady clocks only after some 15 ms of
    # continuous work (a cold start measured 201-202 us per decode step over the first 60 steps,
    # 192 us afterwards), and the decode step is timed right after them, before the prefill legs.
    if not args.no_checkpoint_copy:
        legs["checkpoint_copy"] = checkpoint_copy_leg(pool, dev, stream, e0, e1)
    if not args.no_int8_store:
        legs["int8_checkpoint_store"] = int8_store_leg(pool, sh, dev, stream, e0, e1)
    if not args.no_multi_decode:
        legs["multi_token_decode"] = multi_token_decode(dev, stream, e0, e1, w)
    if not args.no_mamba1:
        legs["mamba1_decode"] = mamba1_decode(dev, stream, e0, e1)
        legs["mamba1_prefill"] = mamba1_prefill_leg(dev, stream, e0, e1)

    # W untimed steps; the last of them is queued after the barrier, ahead of the first event, so
    # that the GPU is not idle while the host enqueues the first timed step
    for _ in range(max(args.warmup - 1, 0)):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    if args.warmup > 0:
        step()
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = e0.elapsed_time(e1) / args.steps
    per_seq = decode_bytes_per_seq(sh)
    launch_bytes = per_seq * batch
    state_bytes = batch * 2 * (sh.nheads * sh.head_dim * sh.d_state * 2 + sh.conv_dim * (sh.conv_kernel - 1) * 2)
    achieved = launch_bytes / (ms * 1e-3) / 1e9
    out = {
        "metric": "decode tokens/s and state GB/s (% of HBM peak); prefill tokens/s (% MFMA)",
        "value": batch / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": "Mamba2 decode step, Nemotron-H layer shape (H=128, P=64, N=128, G=8, W=4), "
                        "256 live sequences at permuted slots of a 512-slot pool, one token each",
            "batch": batch, "pool_slots": w["num_slots"], "state_dtype": "bf16", "io_dtype": "bf16",
            "parallelism": "single GPU",
        },
        "state_gbps": state_bytes / (ms * 1e-3) / 1e9,
        "wall_s_timed": wall,
        "roofline": {
            "bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS,
            "traffic": measured_traffic(ROOT, "decode_traffic.json", DECODE_SOURCES, "traffic_bytes_per_launch"),
            "kernel": "decode_kernel<bf16, N=128, W=4>", "bytes_per_launch": launch_bytes,
            "bytes_per_sequence": per_seq,
        },
    }

    pw = None
    if not args.no_prefill:
        pw = synth.prefill_workload(2)
        legs["prefill"] = prefill_leg(pw, dev, stream, e0, e1)
        if not args.no_prefill_workloads:
            legs["prefill_workloads"] = prefill_workloads(dev, stream, e0, e1)
    if "checkpoint_copy" in legs:
        # the copy is also the measured ceiling a streaming kernel reaches on this part
        out["roofline"]["copy_ceiling_gbs"] = legs["checkpoint_copy"]["gbs"]
        out["roofline"]["frac_of_copy_ceiling"] = achieved / legs["checkpoint_copy"]["gbs"]
    if "multi_token_decode" in legs:
        legs["multi_token_decode"]["speedup_vs_single_steps"] = 4 * ms / legs["multi_token_decode"]["ms"]
    out.update(legs)

    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, pw, args.cpu_seconds)

    print(json.dumps(out), flush=True)
    return 0


def checkpoint_copy_leg(pool, dev, stream, e0, e1) -> dict:
    """COPY_PAIRS slot-to-slot copies of both state objects, slots [0, 256) -> [256, 512) of the
    decode pool; also the measured streaming ceiling of the part (a copy of known size)."""
    import torch
    n = COPY_PAIRS
    src = torch.arange(0, n, device=dev, dtype=torch.int32)
    dst = torch.arange(n, 2 * n, device=dev, dtype=torch.int32)
    cms = time_calls(lambda: pool.checkpoint(0, src, dst), 2, 10, stream, e0, e1)
    ssm_b, conv_b = pool.info()
    moved = 2 * n * (ssm_b + conv_b)
    gbs = moved / (cms * 1e-3) / 1e9
    return {"workload": f"{n} slot-to-slot copies of both state objects (bf16, {ssm_b + conv_b} B per slot)",
            "ms": cms, "copies_per_s": n / (cms * 1e-3), "bytes_per_launch": moved, "gbs": gbs,
            "hbm_frac": gbs / HBM_PEAK_GBS}


def int8_store_leg(pool, sh, dev, stream, e0, e1) -> dict:
    """int8 checkpoint store: 256 slots quantized into 256 entries, and restored into the other half."""
    import torch
    n = COPY_PAIRS
    store = pool.int8_store(n)
    sl = torch.arange(0, n, device=dev, dtype=torch.int32)
    ent = torch.arange(0, n, device=dev, dtype=torch.int32)
    dst = torch.arange(n, 2 * n, device=dev, dtype=torch.int32)
    ssm_b, conv_b = pool.info()
    codes_b = ssm_b // 2
    scales_b = sh.nheads * sh.d_state * 4
    put_bytes = n * (ssm_b + codes_b + scales_b + 2 * conv_b)       # read state + window, write entry
    get_bytes = n * (codes_b + scales_b + ssm_b + 2 * conv_b)       # read entry, write state + window
    res = {}
    for name, fn, nbytes in (("put", lambda: pool.int8_put(store, 0, sl, ent), put_bytes),
                             ("get", lambda: pool.int8_get(store, 0, ent, dst), get_bytes)):
        t = time_calls(fn, 2, 10, stream, e0, e1)
        res[name] = {"ms": t, "states_per_s": n / (t * 1e-3), "bytes_per_launch": nbytes,
                     "gbs": nbytes / (t * 1e-3) / 1e9, "hbm_frac": nbytes / (t * 1e-3) / 1e9 / HBM_PEAK_GBS}
    res["workload"] = (f"{n} bf16 slots quantized into int8 store entries (put) and restored into fresh "
                       "slots (get), Nemotron-H layer shape")
    res["entry_bytes"] = codes_b + scales_b + conv_b
    res["slot_bytes"] = ssm_b + conv_b
    del store
    return res


def prefill_leg(pw, dev, stream, e0, e1) -> dict:
    """Chunked prefill of one 8192-token sequence (chunk 256) at the Nemotron-H layer shape, bf16
    state, zero initial state, final state and window into slot 17."""
    import torch

    from recurrent_state_update_amd import synth
    from recurrent_state_update_amd.pool import LayerWeights, Pool
    psh = pw["shape"]
    ppool = Pool.allocate(1, 32, psh.nheads, psh.head_dim, psh.d_state, psh.n_groups, psh.conv_kernel,
                          torch.bfloat16, torch.bfloat16, dev)
    PW = LayerWeights.from_numpy(pw["params"], dev)
    pu = synth.to_torch(pw["u"], "bf16").to(dev)
    pz = synth.to_torch(pw["z"], "bf16").to(dev)
    pdt = synth.to_torch(pw["dt"], "bf16").to(dev)
    T = pu.shape[0]
    py = torch.empty((T, psh.intermediate), dtype=torch.bfloat16, device=dev)
    px, pB, pC = ppool.split_xbc(pu)
    ws = torch.empty(ppool.workspace_size(pw["cu_seqlens"], pw["chunk"]), dtype=torch.uint8, device=dev)

    def pstep():
        ppool.prefill(0, PW, pw["cu_seqlens"], [17], [0], px, pB, pC, pz, pdt, py,
                      chunk_size=pw["chunk"], workspace=ws)

    pms = time_calls(pstep, 3, 10, stream, e0, e1)
    flops = prefill_dense_flops_per_token(psh, pw["chunk"]) * T
    io_bytes = T * (psh.conv_dim + psh.intermediate + psh.nheads + psh.intermediate) * 2 \
        + psh.nheads * psh.head_dim * psh.d_state * 2 + psh.conv_dim * 3 * 2
    res = {
        "workload": "chunked prefill of one 8192-token sequence, chunk 256, same layer shape, bf16 state",
        "ms": pms, "tokens_per_s": T / (pms * 1e-3),
        "mfma_dense_tflops": flops / (pms * 1e-3) / 1e12,
        "mfma_frac": flops / (pms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS,
        "hbm_algorithmic_gbs": io_bytes / (pms * 1e-3) / 1e9,
        "hbm_frac": io_bytes / (pms * 1e-3) / 1e9 / HBM_PEAK_GBS,
    }
    # bytes the kernels move per call, intermediates included, from the committed counter record
    ptraffic = measured_traffic(ROOT, "prefill_traffic.json", PREFILL_SOURCES, "traffic_bytes_per_call")
    res["traffic"] = ptraffic
    if ptraffic is not None:
        res["traffic_gbs"] = ptraffic / (pms * 1e-3) / 1e9
        res["traffic_frac"] = ptraffic / (pms * 1e-3) / 1e9 / HBM_PEAK_GBS
    del ppool, ws
    torch.cuda.empty_cache()
    return res


def multi_token_decode(dev, stream, e0, e1, w) -> dict:
    """Speculative decode step: the 256 sequences of the decode workload with 4 tokens each (a
    verified token and 3 drafts), the state after every token kept in a slot of its own (a
    1280-slot bf16 pool).  Algorithmic bytes per sequence: one state and window read, four written,
    and the io of four tokens."""
    import torch

    from recurrent_state_update_amd.pool import LayerWeights, Pool
    sh = w["shape"]
    K, n = 4, len(w["slots"])
    gen = torch.Generator(device=dev).manual_seed(11)
    pool = Pool.allocate(1, n * (K + 1), sh.nheads, sh.head_dim, sh.d_state, sh.n_groups, sh.conv_kernel,
                         torch.bfloat16, torch.bfloat16, dev)
    pool.ssm.normal_(0.0, 0.1, generator=gen)
    pool.conv.normal_(0.0, 0.1, generator=gen)
    perm = torch.randperm(n * (K + 1), generator=gen, device=dev).to(torch.int32)
    ins, outs = perm[:n].contiguous(), perm[n:].reshape(n, K).contiguous()
    u = torch.randn((n * K, sh.conv_dim), generator=gen, device=dev).bfloat16()
    z = torch.randn((n * K, sh.intermediate), generator=gen, device=dev).bfloat16()
    dt = torch.randn((n * K, sh.nheads), generator=gen, device=dev).bfloat16()
    y = torch.empty((n * K, sh.intermediate), dtype=torch.bfloat16, device=dev)
    W = LayerWeights.from_numpy(w["params"], dev)
    x, B, C = pool.split_xbc(u)
    step = lambda: pool.decode_multi(0, W, ins, outs, x, B, C, z, dt, y)
    t = time_calls(step, 5, 50, stream, e0, e1)
    ssm_b, conv_b = pool.info()
    io = (sh.conv_dim + sh.intermediate + sh.nheads + sh.intermediate) * 2
    nbytes = n * ((1 + K) * (ssm_b + conv_b) + K * io)
    del pool
    torch.cuda.empty_cache()
    return {"workload": f"{n} sequences x {K} tokens (a verified token and {K - 1} drafts), state after every "
                        "token kept, Nemotron-H layer shape, bf16 state",
            "ms": t, "tokens_per_s": n * K / (t * 1e-3), "bytes_per_launch": nbytes,
            "gbs": nbytes / (t * 1e-3) / 1e9, "hbm_frac": nbytes / (t * 1e-3) / 1e9 / HBM_PEAK_GBS}


def mamba1_decode(dev, stream, e0, e1) -> dict:
    """The pool's second state family: a Mamba1 decode step (D = 8192, N = 16, conv 4) for 256
    sequences at permuted slots of a 512-slot bf16 pool.  Algorithmic bytes per sequence: the
    (D, N) state and the (D, 3) window read and written, x, z, dt, B, C in and y out."""
    import torch

    from recurrent_state_update_amd import synth
    from recurrent_state_update_amd.pool import LayerWeights, Pool
    D, N, Wd = synth.MAMBA1_D, synth.MAMBA1_N, synth.MAMBA1_W
    n = 256
    rng = np.random.default_rng(12)
    gen = torch.Generator(device=dev).manual_seed(12)
    pool = Pool.allocate_mamba1(1, 2 * n, D, N, Wd, torch.bfloat16, torch.bfloat16, dev)
    pool.ssm.normal_(0.0, 0.1, generator=gen)
    pool.conv.normal_(0.0, 0.1, generator=gen)
    W = LayerWeights.from_numpy(synth.mamba1_layer_params(rng, D, N, Wd), dev)
    sl = torch.from_numpy(rng.permutation(2 * n)[:n].astype(np.int32)).to(dev)
    x, z, dt = (torch.randn((n, D), generator=gen, device=dev).bfloat16() for _ in range(3))
    B, C = (torch.randn((n, N), generator=gen, device=dev).bfloat16() for _ in range(2))
    y = torch.empty((n, D), dtype=torch.bfloat16, device=dev)
    step = lambda: pool.mamba1_decode_step(0, W, sl, x, B, C, z, dt, y)
    t = time_calls(step, 10, 200, stream, e0, e1)
    ssm_b, conv_b = pool.info()
    per_seq = 2 * (ssm_b + conv_b) + (3 * D + 2 * N) * 2 + D * 2
    del pool
    torch.cuda.empty_cache()
    return {"workload": f"Mamba1 decode step, D={D}, N={N}, conv {Wd}, {n} sequences at permuted slots of a "
                        f"{2 * n}-slot bf16 pool",
            "ms": t, "tokens_per_s": n / (t * 1e-3), "bytes_per_launch": n * per_seq,
            "gbs": n * per_seq / (t * 1e-3) / 1e9, "hbm_frac": n * per_seq / (t * 1e-3) / 1e9 / HBM_PEAK_GBS}


def mamba1_prefill_leg(dev, stream, e0, e1) -> dict:
    """Mamba1 prefill (D = 8192, N = 16, conv 4, bf16 state and rows) of 8 sequences of 1024 rows
    from zero states, chunking chosen by the library (here one chunk per sequence, so only the
    output launch has work).  Algorithmic bytes per row: x, z, dt and y of D and B, C of N at
    2 bytes; the (D, N) state and window written once per sequence.  The recurrence takes one
    exponential per (row, channel, state index)."""
    import torch

    from recurrent_state_update_amd import synth
    from recurrent_state_update_amd.pool import LayerWeights, Pool
    D, N, Wd = synth.MAMBA1_D, synth.MAMBA1_N, synth.MAMBA1_W
    ns, ln, Q = 8, 1024, 0
    T = ns * ln
    rng = np.random.default_rng(13)
    gen = torch.Generator(device=dev).manual_seed(13)
    pool = Pool.allocate_mamba1(1, ns, D, N, Wd, torch.bfloat16, torch.bfloat16, dev)
    W = LayerWeights.from_numpy(synth.mamba1_layer_params(rng, D, N, Wd), dev)
    x, z, dt = (torch.randn((T, D), generator=gen, device=dev).bfloat16() for _ in range(3))
    B, C = (torch.randn((T, N), generator=gen, device=dev).bfloat16() for _ in range(2))
    y = torch.empty((T, D), dtype=torch.bfloat16, device=dev)
    cu = np.arange(ns + 1, dtype=np.int32) * ln
    slots = np.arange(ns, dtype=np.int32)
    zeros = np.zeros(ns, np.uint8)
    ws = torch.empty(pool.mamba1_workspace_size(ns, T, Q), dtype=torch.uint8, device=dev)
    step = lambda: pool.mamba1_prefill(0, W, cu, slots, zeros, x, B, C, z, dt, y, chunk_size=Q, workspace=ws)
    t = time_calls(step, 3, 20, stream, e0, e1)
    ssm_b, conv_b = pool.info()
    nbytes = T * (4 * D + 2 * N) * 2 + ns * (ssm_b + conv_b)
    del pool, ws
    torch.cuda.empty_cache()
    return {"workload": f"Mamba1 prefill, D={D}, N={N}, conv {Wd}, {ns} sequences x {ln} rows from zero "
                        f"states, chunking chosen by the library (one chunk per sequence), bf16 state and rows",
            "ms": t, "tokens_per_s": T / (t * 1e-3), "bytes_per_launch": nbytes,
            "gbs": nbytes / (t * 1e-3) / 1e9, "hbm_frac": nbytes / (t * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "exp_per_s": T * D * N / (t * 1e-3)}


def prefill_workloads(dev, stream, e0, e1) -> dict:
    """The mixed continuous batch (32 varlen prefills with checkpoints every 1024 tokens plus 224
    single-token decodes, bf16 state: both launches on one stream, and each part alone) and the
    long context (2 x 131072 tokens through 48 independently parameterised layers, fp32 state).
    Layouts and parameters come from the workload generators; token values and live decode states
    are drawn on the GPU (they do not affect the timing)."""
    import torch

    from recurrent_state_update_amd import synth
    from recurrent_state_update_amd.pool import LayerWeights, Pool
    sh = synth.NEMOTRON_H
    gen = torch.Generator(device=dev).manual_seed(7)

    def tokens(T, y_dtype):
        u = torch.randn(T, sh.conv_dim, device=dev, generator=gen).bfloat16()
        z = torch.randn(T, sh.intermediate, device=dev, generator=gen).bfloat16()
        dt = torch.randn(T, sh.nheads, device=dev, generator=gen).bfloat16()
        return u, z, dt, torch.empty(T, sh.intermediate, device=dev, dtype=y_dtype)

    def timed(fn, reps, warm=2):
        return time_calls(fn, warm, reps, stream, e0, e1)

    res = {}
    _, params, lens, p_slots, d_slots, ck = synth.mixed_layout(3)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T, nd = int(cu[-1]), len(d_slots)
    pool = Pool.allocate(1, 512, sh.nheads, sh.head_dim, sh.d_state, sh.n_groups, sh.conv_kernel,
                         torch.bfloat16, torch.bfloat16, dev)
    pool.ssm.normal_(0.0, 0.1, generator=gen)
    pool.conv.normal_(0.0, 0.1, generator=gen)
    W = LayerWeights.from_numpy(params, dev)
    u, z, dt, y = tokens(T, torch.bfloat16)
    x, B, C = pool.split_xbc(u)
    du, dz, ddt, dy = tokens(nd, torch.bfloat16)
    dx, dB, dC = pool.split_xbc(du)
    dsl = torch.from_numpy(d_slots).to(dev)
    ws = torch.empty(pool.workspace_size(cu, 256, ckpt_interval=1024, ckpt_slots=ck), dtype=torch.uint8, device=dev)

    def pre():
        pool.prefill(0, W, cu, p_slots, np.zeros(len(lens), np.uint8), x, B, C, z, dt, y, chunk_size=256,
                     ckpt_interval=1024, ckpt_slots=ck, workspace=ws)

    def dec():
        pool.decode_step(0, W, dsl, dx, dB, dC, dz, ddt, dy)

    def both():
        pre()
        dec()

    ms_p, ms_d, ms = timed(pre, 10), timed(dec, 10), timed(both, 10)
    res["mixed_batch"] = {"workload": f"{len(lens)} varlen prefills of U(128, 4096) tokens ({T} in all), chunk 256, "
                                      f"checkpoints every 1024 tokens, plus {nd} single-token decodes, one stream, "
                                      "bf16 state",
                          "ms": ms, "tokens_per_s": (T + nd) / (ms * 1e-3),
                          "prefill_ms": ms_p, "prefill_tokens_per_s": T / (ms_p * 1e-3),
                          "decode_ms": ms_d, "decode_tokens_per_s": nd / (ms_d * 1e-3)}
    del pool, ws, u, z, dt, y, x, B, C, du, dz, ddt, dy, dx, dB, dC
    torch.cuda.empty_cache()

    lw = synth.long_workload()
    T, nl = lw["seqs"] * lw["L"], lw["num_layers"]
    pool = Pool.allocate(nl, lw["seqs"], sh.nheads, sh.head_dim, sh.d_state, sh.n_groups, sh.conv_kernel,
                         torch.float32, torch.bfloat16, dev)
    Ws = [LayerWeights.from_numpy(synth.long_layer_params(layer), dev) for layer in range(nl)]
    u, z, dt, y = tokens(T, torch.float32)
    x, B, C = pool.split_xbc(u)
    ws = torch.empty(pool.workspace_size(lw["cu_seqlens"], lw["chunk"]), dtype=torch.uint8, device=dev)

    def stack():
        for layer in range(nl):
            pool.prefill(layer, Ws[layer], lw["cu_seqlens"], lw["slots"], lw["has_init"], x, B, C, z, dt, y,
                         chunk_size=lw["chunk"], workspace=ws)

    ms = timed(stack, 2, warm=1)
    res["long_context_fp32"] = {"workload": f"{lw['seqs']} x {lw['L']} tokens through {nl} layer calls, chunk 256, "
                                            "fp32 state",
                                "ms": ms, "tokens_per_s": T / (ms * 1e-3),
                                "ms_per_layer": ms / nl, "layer_tokens_per_s": T / (ms / nl * 1e-3)}
    del pool, ws, u, z, dt, y, x, B, C
    torch.cuda.empty_cache()
    return res


def cpu_baseline(w, pw, budget_s: float) -> dict:
    """The fp64 CPU oracle, as it stands, on bounded samples of the benchmark workloads, on one host
    thread (numpy with its thread pool limited to one): the decode step at the Nemotron-H layer
    shape (whole 256-sequence steps, repeated while the budget lasts), and the prefill of one
    8192-token sequence and of the 2 x 131072-token fp32-state long context, each on its first 256
    tokens with all 128 heads (the oracle's cost per token does not depend on the position)."""
    from threadpoolctl import threadpool_limits

    from oracle import mamba2 as orc
    from recurrent_state_update_amd import synth
    host_cores = len(os.sched_getaffinity(0))
    sh = w["shape"]
    n = len(w["slots"])
    per = {}
    with threadpool_limits(limits=1):
        done, el = 0, 0.0
        while el < budget_s:
            # 16 sequences of the step at a time; the oracle's pool copy is set up outside the timing
            idx = np.arange(done % n, min(done % n + 16, n))
            ref = orc.PoolRef(sh, 1, len(idx), "bf16", "bf16")
            ref.ssm[0], ref.conv[0] = w["ssm0"][idx], w["conv0"][idx]
            t0 = time.perf_counter()
            orc.decode_step(ref, 0, w["params"], np.arange(len(idx)), w["u"][idx], w["z"][idx], w["dt"][idx], "bf16")
            el += time.perf_counter() - t0
            done += len(idx)
        per["decode_256seq"] = {"tokens_per_s": done / el, "seconds": el,
                                "sample": f"{done} decode tokens of the 256-sequence step, 16 sequences per call"}
        k = 256
        if pw is not None:
            ref = orc.PoolRef(pw["shape"], 1, 32, "bf16", "bf16")
            t0 = time.perf_counter()
            orc.prefill(ref, 0, pw["params"], [0, k], [17], [0], [0], pw["u"][:k], pw["z"][:k], pw["dt"][:k], "bf16")
            el = time.perf_counter() - t0
            per["prefill_8192tok"] = {"tokens_per_s": k / el, "seconds": el,
                                      "sample": f"first {k} of the 8192 tokens, all 128 heads, bf16 state"}
        lw = synth.long_workload()
        bu, bz, bdt = synth.long_token_block(0)
        ref = orc.PoolRef(lw["shape"], 1, 1, "f32", "bf16")
        t0 = time.perf_counter()
        orc.prefill(ref, 0, synth.long_layer_params(0), [0, k], [0], [0], [0], bu[:k], bz[:k], bdt[:k], "f32")
        el = time.perf_counter() - t0
        per["long_context_fp32"] = {"tokens_per_s": k / el, "seconds": el,
                                    "sample": f"first {k} tokens of sequence 0 in layer 0, all 128 heads, fp32 "
                                              "state; the whole workload is 2 x 131072 tokens x 48 layers"}
    d = per["decode_256seq"]
    return {"value": d["tokens_per_s"], "unit": "tokens/s", "cores": 1, "threads": 1, "workers": 1,
            "host_cores": host_cores, "kind": "oracle",
            "sample": f"{d['sample']} ({d['seconds']:.1f} s) on one host thread, numpy fp64; per-workload "
                      "samples in per_workload",
            "per_workload": per}


if __name__ == "__main__":
    sys.exit(main())
