#!/usr/bin/env python3
"""Benchmark of the 3D-RoPE video-DiT attention layer on one MI355X.

One step = one pass of the layer's hot path over one batch of synthetic
inputs already resident in HBM: fused per-head RMSNorm + 3D-RoPE of q and k
(vdit_rope_qk), then exact FULL softmax attention (vdit_attn_fwd), on the
Wan-1.3B-shaped layer: latent grid 21 x 30 x 52 = 32760 tokens, 12 heads,
head_dim 128, bf16, RoPE split 22/21/21 pairs.

Prints ONE JSON line.  `value` is attention TFLOP/s over the whole step
(matmul FLOPs 4 L^2 D H per layer; exps not counted).  `roofline` reports the
attention kernel alone, timed with HIP events on the stream it runs on;
`cpu_baseline` times the fp64 oracle on a bounded sample (run before the GPU
is touched, over a process pool of the host's cores, one head per task).

  python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu-baseline]
                                 (K, W default to 50, 10)
  python bench.py --workload N   (the other workloads, one JSON line each,
                                  with their own cpu_baseline; K and W
                                  default to at least 100 ms of steps each)
  python bench.py --calibrate-copy | --traffic-from DIR | --kernel-stats-from DIR
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBPS = 8000.0      # MI355X HBM3E
METRIC = "attention TFLOP/s and ms/layer on 1 MI355X (% of bf16 MFMA peak)"
ATTN_SRC = os.path.join(ROOT, "video_diffusion_transformer_rmsnorm_amd", "csrc", "attn_mfma.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_fwd_wan13b_traffic.json")
PROBES_LIB = os.path.join(ROOT, "video_diffusion_transformer_rmsnorm_amd", "libvdit_probes.so")
MALL_BYTES = 256 << 20      # memory-side Infinity Cache


def src_hash(path: str) -> str:
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def measured_traffic():
    """HBM bytes per attention launch from the committed rocprofv3 --pmc summary,
    or None if absent or taken on a different kernel source."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_sha256_16") != src_hash(ATTN_SRC):
        return None
    return t.get("hbm_bytes_per_launch")


# ------------------------------------------------------------ CPU baseline --
# The oracle (oracle/, float64 numpy, as it stands) on a bounded sample of the
# workload, one head per task over a pool of forked worker processes, each
# with single-threaded BLAS, so `cores` is the number of processes that ran.
# It runs before the GPU is initialised (forking a process that holds a GPU
# context is avoided), on the same seeded inputs the GPU run uses.

_CPU = {}  # inputs of the current baseline, inherited by the forked workers


def _one_blas_thread():
    from threadpoolctl import threadpool_limits
    _CPU["_limit"] = threadpool_limits(1)


def _pool_map(fn, items):
    import multiprocessing as mp
    n = min(len(os.sched_getaffinity(0)), 16, len(items))
    with mp.get_context("fork").Pool(n, initializer=_one_blas_thread) as pool:
        out = pool.map(fn, items)
    return out, n


def _head(t, h):
    return t[:, :, h:h + 1]


ROW_BLOCK = 2048  # query rows per oracle attention call (bounds its score matrix to ~0.5 GB)


def _task_full(h):
    import oracle as O
    c = _CPU
    wq, wk = O.rope_qk(_head(c["q"], h), _head(c["k"], h), c["grid"], c["pairs"])
    v = _head(c["v"], h)
    rows = c["rows"]
    for i in range(0, len(rows), ROW_BLOCK):
        O.attention(wq[:, rows[i:i + ROW_BLOCK]], wk, v)


def _task_ring(h):
    import oracle as O
    c = _CPU
    q0, nq = c["q_range"]
    wq, wk = O.rope_qk(_head(c["q"], h), _head(c["k"], h), c["grid"], c["pairs"])
    qs = wq[:, q0 + c["rows"]]
    v = _head(c["v"], h)
    O.ring_attention(qs, [wk[:, s:s + n] for s, n in c["chunks"]], [v[:, s:s + n] for s, n in c["chunks"]])


def _task_rolling(h):
    import numpy as np
    import oracle as O
    c = _CPU
    w = c["w"]
    kh = h // (w.heads // w.kv_heads)
    q, k, v = c["q"][:, :, h:h + 1], c["k"][:, :, kh:kh + 1], c["v"][:, :, kh:kh + 1]
    for f in c["frames"]:
        win = list(O.rolling_window(f, w.n_slots))
        f0, T = win[0], w.grid[0]
        ks, vs = [], []
        for u in win:
            _, ku = O.rope_qk(k[u][None], k[u][None], w.grid, w.pairs, t_offset=T * (u - f0))
            ks.append(ku)
            vs.append(O.rmsnorm(v[u][None]) if w.kv_norm else v[u][None])
        qr, _ = O.rope_qk(q[f][None], q[f][None], w.grid, w.pairs, t_offset=T * (f - f0),
                          q_norm=False if w.kv_norm else None)
        O.attention(qr[:, c["rows"]], np.concatenate(ks, 1), np.concatenate(vs, 1))


def _task_hybrid(h):
    import oracle as O
    c = _CPU
    w = c["w"]
    wq, wk = O.rope_qk(_head(c["q"], h), _head(c["k"], h), w.grid, w.pairs)
    o_s, l_s, o_l, l_l = O.hybrid_partials(wq, wk, _head(c["v"], h), w.chunk_tokens, overlap=w.overlap_tokens)
    O.lse_merge(o_s, l_s, o_l, l_l)


def cpu_baseline(w, rows: int = 32760, seed: int = 99):
    """Time the oracle on a bounded sample of workload w; returns the
    cpu_baseline object (value in the benchmark line's unit, TFLOP/s of the
    sample's attention matmuls)."""
    import numpy as np
    import workloads as WL
    q, k, v = WL.workload_inputs(w)
    _CPU.clear()
    _CPU.update(q=q.values, k=k.values, v=v.values, grid=w.grid, pairs=w.pairs, w=w)
    heads = list(range(w.heads))
    if w.mode == "full":
        r = np.arange(w.tokens) if rows >= w.tokens else WL.sample_rows(w.tokens, rows, seed)
        _CPU["rows"] = r
        fn, flops = _task_full, WL.flops_full(len(r), w.tokens, w.heads, w.head_dim)
        sample = (f"{len(r)} of {w.tokens} query rows x {w.heads} heads vs all {w.tokens} keys "
                  f"(oracle attention on blocks of {ROW_BLOCK} rows), plus RMSNorm+RoPE of every token")
    elif w.mode == "ring":
        q0, nq = w.q_range
        r = WL.sample_rows(nq, min(rows, 4096), seed)
        _CPU.update(rows=r, q_range=w.q_range, chunks=w.kv_chunks)
        lkv = sum(n for _, n in w.kv_chunks)
        fn, flops = _task_ring, WL.flops_full(len(r), lkv, w.heads, w.head_dim)
        sample = (f"{len(r)} of {nq} query rows x {w.heads} heads vs {len(w.kv_chunks)} chunks "
                  f"({lkv} keys), per-chunk attention merged by LSE, plus RMSNorm+RoPE")
    elif w.mode == "rolling":
        frames = list(range(w.n_slots, min(w.n_frames, w.n_slots + 4)))
        r = WL.sample_rows(w.tokens, min(rows, 2048), seed)
        _CPU.update(rows=r, frames=frames)
        fn = _task_rolling
        flops = len(frames) * WL.flops_full(len(r), w.tokens * w.n_slots, w.heads, w.head_dim)
        sample = (f"decode steps {frames[0]}..{frames[-1]} (full window of {w.n_slots}): {len(r)} of "
                  f"{w.tokens} query rows x {w.heads} heads vs {w.tokens * w.n_slots} keys, plus the "
                  "window's RMSNorm+RoPE")
    else:
        fn, flops = _task_hybrid, WL.hybrid_flops(w)
        sample = (f"the whole call: {w.tokens} tokens x {w.heads} heads, chunks of {w.chunk_tokens}"
                  f" (overlap {w.overlap_tokens}), softmax and linear partials, plus RMSNorm+RoPE")
    t0 = time.perf_counter()
    _, n = _pool_map(fn, heads)
    dt = time.perf_counter() - t0
    _CPU.clear()
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": n, "kind": "oracle",
            "sample": f"{sample}; one head per task on {n} processes; {dt:.1f} s wall",
            "seconds": round(dt, 2), "host_cpus": len(os.sched_getaffinity(0))}


# ------------------------------------------------------------------ timing --

def _up(t, dev):
    import numpy as np
    import torch
    if t.dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(t.bits).view(np.int16)).view(torch.bfloat16).to(dev)
    return torch.from_numpy(t.values.astype(np.float32)).to(dev)


def _time_steps(step, steps, warmup, warm_ms: float = 100.0, timed_ms: float = 100.0):
    """Run warmup calls of step(i), then `steps` timed calls back to back,
    nothing else on the stream between them; returns (wall ms per step of
    those, sorted per-step HIP-event ms on torch's current stream from a
    second pass of `steps` calls with an event pair around each, steps,
    warmup).  The events stay out of the first pass: on steps of ~0.1 ms
    their records add ~10% to the wall clock.

    `steps` / `warmup` None: sized from the first five warm-up calls to at
    least timed_ms of timed work (at least 50 steps) and warm_ms of warm-up
    (at least 10 steps).  After an idle spell the clock takes milliseconds
    to come up: with 10 warm-up steps of 0.1 ms the first 50 timed ones ran
    15% slower than the next 50."""
    import torch
    stream = torch.cuda.current_stream()
    done = 0
    if steps is None or warmup is None:
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(5):
            step(i)
        torch.cuda.synchronize()
        done = 5
        per = max((time.perf_counter() - t0) * 1e3 / done, 1e-3)
        warmup = max(10, done + math.ceil(warm_ms / per)) if warmup is None else warmup
        steps = max(50, math.ceil(timed_ms / per)) if steps is None else steps
    for i in range(done, warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(warmup + i)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3 / steps
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for i, e in enumerate(evs):
        e[0].record(stream)
        step(warmup + steps + i)
        e[1].record(stream)
    torch.cuda.synchronize()
    return wall, sorted(a.elapsed_time(b) for a, b in evs), steps, max(warmup, done)


def key_norm_bound(head_dim: int) -> float:
    """Bound on the norm of keys RMS-normalised with gain 1 and stored in
    bf16: sqrt(head_dim), widened for the rounding of each element."""
    return math.sqrt(head_dim) * (1.0 + 2.0 ** -7)


def bench_full(args):
    import torch
    import video_diffusion_transformer_rmsnorm_amd as V
    import workloads as WL

    w = WL.WORKLOADS[2]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    q, k, v = WL.workload_inputs(w)
    qd, kd, vd = _up(q, dev), _up(k, dev), _up(v, dev)
    del q, k, v
    # two input sets for the RMSNorm + RoPE, used alternately: each step's
    # rotation reads q, k that the previous step did not touch
    qd2, kd2 = qd.clone(), kd.clone()
    qr, kr = torch.empty_like(qd), torch.empty_like(kd)
    o = torch.empty_like(qd)
    lse = torch.empty((1, w.heads, w.tokens), dtype=torch.float32, device=dev)
    grid = V.make_grid(*w.grid, w.pairs)
    stream = torch.cuda.current_stream()

    # the step's keys come out of vdit_rope_qk RMS-normalised (gain 1): their
    # norms are at most sqrt(D) up to bf16 rounding, which lets the attention
    # call skip its own pass over the keys (same results, see vdit.h)
    knorm = key_norm_bound(w.head_dim)
    evs = {}

    def step(i):
        e = evs.get(i)
        if e is not None:
            e[0].record(stream)
        src = (qd, kd) if i % 2 == 0 else (qd2, kd2)
        V.vdit_rope_qk(src[0], src[1], grid, q_out=qr, k_out=kr)
        if e is not None:
            e[1].record(stream)
        V.vdit_attn_fwd(qr, kr, vd, o=o, lse=lse, key_norm_max=knorm)
        if e is not None:
            e[2].record(stream)

    for i in range(args.warmup, args.warmup + args.steps):
        evs[i] = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    ms_step, _, _, _ = _time_steps(step, args.steps, args.warmup)
    rope_each = [e[0].elapsed_time(e[1]) for e in evs.values()]
    attn_each = sorted(e[1].elapsed_time(e[2]) for e in evs.values())
    rope_ms = sum(rope_each) / args.steps
    attn_ms = sum(attn_each) / args.steps
    flops = WL.flops_full(w.tokens, w.tokens, w.heads, w.head_dim)
    rope_bytes = 2 * 2 * w.tokens * w.heads * w.head_dim * 2  # q,k read + write, bf16
    achieved = flops / (attn_ms * 1e-3) / 1e12
    del qd2, kd2
    out = {
        "metric": METRIC,
        "value": round(flops / (ms_step * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1), bf16 RNE)",
        "config": {"workload": "wan1.3b_full_layer_21x30x52", "tokens": w.tokens, "heads": w.heads,
                   "head_dim": w.head_dim, "rope_pairs": list(w.pairs), "mode": "full",
                   "step": "rmsnorm+3d_rope(q,k) -> full attention", "parallelism": "none (1 GPU)"},
        "attn_ms": round(attn_ms, 4),
        "attn_ms_median": round(attn_each[len(attn_each) // 2], 4),
        "attn_ms_min": round(attn_each[0], 4),
        "rope_ms": round(rope_ms, 4),
        "pct_bf16_peak_step": round(100 * flops / (ms_step * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 2),
        "rope_GBps": round(rope_bytes / (rope_ms * 1e-3) / 1e9, 1),
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": measured_traffic(), "kernel": "attn_mfma_kernel<128,8,1,false,2>",
                     "algorithmic_flops_per_launch": flops},
    }
    del qr, kr, o, lse
    if not args.no_peaks:
        out["rope_rotated"] = rope_rotated(w, qd, kd, grid)
        out["measured_peaks"] = measured_peaks(achieved, out["rope_rotated"]["GBps"])
    return out


def rope_rotated(w, qd, kd, grid, reps: int = 24):
    """RMSNorm + RoPE alone over enough distinct buffer sets (inputs and
    outputs) that consecutive calls touch more than twice the 256 MB
    memory-side cache: the call's HBM rate with no cache residency."""
    import torch
    import video_diffusion_transformer_rmsnorm_amd as V
    per = 4 * qd.numel() * qd.element_size()  # q, k in + out
    nsets = max(2, math.ceil(2 * MALL_BYTES / per) + 1)
    sets = [(qd.clone(), kd.clone(), torch.empty_like(qd), torch.empty_like(kd)) for _ in range(nsets)]

    def step(i):
        a, b, c, d = sets[i % nsets]
        V.vdit_rope_qk(a, b, grid, q_out=c, k_out=d)

    _, each, _, _ = _time_steps(step, reps, nsets)
    ms = sum(each) / len(each)
    del sets
    torch.cuda.empty_cache()
    return {"ms": round(ms, 4), "GBps": round(per / (ms * 1e-3) / 1e9, 1), "buffer_sets": nsets,
            "bytes_per_call": per, "frac_of_hbm_peak": round(per / (ms * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4)}


def mfma_peak(reps: int = 3, iters: int = 20000):
    """Sustained bf16 matrix-core rate from the probe kernel (libvdit_probes.so):
    back-to-back v_mfma_f32_32x32x16_bf16 from registers at two wavefronts
    per SIMD, on random-data operands (eight pairs in turn) and on one
    constant pair; None if the probe is not built."""
    import ctypes
    import torch
    if not os.path.exists(PROBES_LIB):
        return None
    lib = ctypes.CDLL(PROBES_LIB)
    lib.vdit_probe_mfma_peak.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                                         ctypes.c_int, ctypes.c_void_p]
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    blocks = 2 * cus  # 8 wavefronts per CU: two per SIMD
    g = torch.Generator().manual_seed(5)
    seed = torch.randn(16 * 64 * 8, generator=g).to(torch.bfloat16).cuda()
    out = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    res = {}
    for vary, name in ((1, "random_operands"), (0, "constant_operands")):
        best = None
        for _ in range(reps + 1):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            rc = lib.vdit_probe_mfma_peak(seed.data_ptr(), out.data_ptr(), iters, vary, blocks, stream.cuda_stream)
            e1.record(stream)
            torch.cuda.synchronize()
            if rc != 0:
                return None
            ms = e0.elapsed_time(e1)
            best = ms if best is None or ms < best else best
        flops = blocks * 4 * iters * 8 * 32768.0
        res[name + "_TFLOPs"] = round(flops / (best * 1e-3) / 1e12, 1)
    return res


def valu_rates(reps: int = 3, iters: int = 20000):
    """Cost of v_exp_f32 in v_sub_f32 issue slots, from the probe kernel
    (libvdit_probes.so): eight independent chains per thread at eight
    wavefronts per SIMD, so that the time is the VALU issue; also an
    exponential and a subtraction per step, to see whether the two overlap.
    None if the probe is not built."""
    import ctypes
    import torch
    if not os.path.exists(PROBES_LIB):
        return None
    lib = ctypes.CDLL(PROBES_LIB)
    if not hasattr(lib, "vdit_probe_valu_rate"):
        return None
    lib.vdit_probe_valu_rate.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    blocks = 8 * cus  # 32 wavefronts per CU: eight per SIMD
    out = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    ms = {}
    for kind in (1, 0, 2):
        best = None
        for _ in range(reps + 1):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            rc = lib.vdit_probe_valu_rate(kind, out.data_ptr(), iters, blocks, stream.cuda_stream)
            e1.record(stream)
            torch.cuda.synchronize()
            if rc != 0:
                return None
            t = e0.elapsed_time(e1)
            best = t if best is None or t < best else best
        ms[kind] = best
    per_simd = blocks * 4 * iters * 8 / (4 * cus)  # chain steps per SIMD
    return {"sub_ns_per_wave_instr_per_simd": round(ms[1] * 1e6 / per_simd, 4),
            "exp_in_sub_slots": round(ms[0] / ms[1], 3),
            "exp_plus_sub_in_sub_slots": round(ms[2] / ms[1], 3)}


def measured_peaks(attn_tflops: float, rope_gbps: float, reps: int = 10):
    """Reference rates measured on the same device after the timed region: the
    matrix-core probe (the ceiling of any bf16 MFMA kernel at this clock and
    power), a bf16 library GEMM (8192^3, hipBLASLt), and a 1 GiB device copy
    as the sustained HBM rate, with the attention and RoPE rates as
    fractions of them (context for the nominal peaks in `roofline`); and the
    cost of the softmax's exponential in plain VALU issue slots."""
    import torch
    out = {}
    mp = mfma_peak()
    if mp:
        out.update({"mfma_probe_" + k: v for k, v in mp.items()})
        out["attn_frac_of_mfma_probe"] = round(attn_tflops / mp["random_operands_TFLOPs"], 4)
    vr = valu_rates()
    if vr:
        out.update({"valu_probe_" + k: v for k, v in vr.items()})
    n = 8192
    a = torch.randn((n, n), device="cuda").to(torch.bfloat16)
    b = torch.randn((n, n), device="cuda").to(torch.bfloat16)
    c = a @ b
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        torch.matmul(a, b, out=c)
    e1.record()
    torch.cuda.synchronize()
    gemm = 2.0 * n ** 3 * reps / (e0.elapsed_time(e1) * 1e-3) / 1e12
    del a, b, c
    nbytes = 1 << 30
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    copy = 2.0 * nbytes * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9
    out.update({"gemm_bf16_8192_TFLOPs": round(gemm, 1), "attn_frac_of_gemm": round(attn_tflops / gemm, 4),
                "copy_1GiB_GBps": round(copy, 1), "rope_rotated_frac_of_copy": round(rope_gbps / copy, 4)})
    return out


def bench_other(args):
    """The other workloads (reference lines, not the headline)."""
    import torch
    import video_diffusion_transformer_rmsnorm_amd as V
    import workloads as WL

    w = WL.WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    q, k, v = WL.workload_inputs(w)
    qd, kd, vd = _up(q, dev), _up(k, dev), _up(v, dev)
    del q, k, v
    grid = V.make_grid(*w.grid, w.pairs)
    extra = {}
    # one scratch area for every attention call of the run, allocated once as
    # a caller would (a workspace may be larger than a call needs)
    ws = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    if w.mode == "ring":
        # the ring step as the shard receives it: per-chunk attention folded
        # into the running partial chunk by chunk (LSE merge in the epilogue);
        # the one-launch form (every chunk resident at once) timed beside it
        # inputs as the layer hands them over: normalised and rotated at their
        # global grid positions (not timed)
        q0, nq = w.q_range
        qq, _ = V.vdit_rope_qk(qd[:, q0:q0 + nq].contiguous(), None, grid, token0=q0)
        kcs = [V.vdit_rope_qk(None, kd[:, s:s + n].contiguous(), grid, token0=s)[1] for s, n in w.kv_chunks]
        vcs = [vd[:, s:s + n].contiguous() for s, n in w.kv_chunks]
        flops = sum(WL.flops_full(nq, n, w.heads, w.head_dim) for _, n in w.kv_chunks)
        knorm = key_norm_bound(w.head_dim)

        def step(i):
            V.vdit_attn_fwd(qq, mode="ring", k_chunks=kcs, v_chunks=vcs, ring_fold=True, key_norm_max=knorm,
                            workspace=ws)

        def step_one(i):
            V.vdit_attn_fwd(qq, mode="ring", k_chunks=kcs, v_chunks=vcs, key_norm_max=knorm, workspace=ws)
        wall1, each1, _, _ = _time_steps(step_one, args.steps, args.warmup)
        extra["one_launch_form"] = {"ms_per_step": round(wall1, 4), "step_ms_median": round(each1[len(each1) // 2], 4),
                                    "TFLOPs": round(flops / (wall1 * 1e-3) / 1e12, 2)}
        # vdit_lse_merge alone on the two chunks' bf16 partials (read 2 x O +
        # 2 x LSE, write O + LSE)
        parts = [V.vdit_attn_fwd(qq, kc_, vc_, key_norm_max=knorm) for kc_, vc_ in zip(kcs, vcs)]
        mo, ml = torch.empty_like(parts[0][0]), torch.empty_like(parts[0][1])
        wall_m, each_m, _, _ = _time_steps(lambda i: V.vdit_lse_merge(parts[0][0], parts[0][1], parts[1][0], parts[1][1],
                                                                o_out=mo, lse_out=ml), args.steps, args.warmup)
        mbytes = 3 * mo.numel() * mo.element_size() + 3 * ml.numel() * 4
        extra["lse_merge"] = {"ms_median": round(each_m[len(each_m) // 2], 4), "bytes": mbytes,
                              "GBps": round(mbytes / (each_m[len(each_m) // 2] * 1e-3) / 1e9, 1)}
        form = "fold: one launch per chunk, LSE merge fused into the epilogue"
    elif w.mode == "rolling":
        kc = torch.zeros((1, w.n_slots, w.tokens, w.kv_heads, w.head_dim), dtype=qd.dtype, device=dev)
        vc = torch.zeros_like(kc)
        for f in range(w.n_slots):
            # the cache starts full of normalised, rotated keys, as the steps leave it
            V.vdit_rope_qk(None, kd[f:f + 1], grid, k_out=kc[:, f])
            vc[:, f].copy_(vd[f:f + 1])
        flops = WL.flops_full(w.tokens, w.tokens * w.n_slots, w.heads, w.head_dim)
        t_step = w.grid[0]
        q_norm = False if w.kv_norm else None
        qbuf = torch.empty_like(qd[:1])

        def frame_step(f):
            # one decode step of stream frame f, in one launch: rotate q
            # (KV-norm: without its norm), normalise and rotate k straight
            # into the cache slot, values into their slot (normalised under
            # KV-norm); then attend
            j, slot = f % w.n_frames, f % w.n_slots
            V.vdit_rope_qkv(qd[j:j + 1], kd[j:j + 1], vd[j:j + 1], grid, q_out=qbuf, k_out=kc[:, slot],
                            v_out=vc[:, slot], t_offset=t_step * f, q_norm=q_norm, v_norm=w.kv_norm)
            V.vdit_attn_fwd(qbuf, mode="rolling", k_cache=kc, v_cache=vc, frame=f,
                            key_norm_max=key_norm_bound(w.head_dim), workspace=ws)

        def step(i):  # steady state: the window is full
            frame_step(w.n_slots + i)

        def stream():
            # the whole stream of n_frames frames from an empty cache (the first
            # n_slots - 1 frames attend to fewer frames)
            for f in range(w.n_frames):
                frame_step(f)
        form = ("decode step: one launch for rope(q), rope(k) into the cache slot and v (normalised under "
                "KV-norm) into its slot, then windowed attention")
    elif w.mode == "hybrid":
        s = torch.zeros((1, w.kv_heads, w.head_dim, w.head_dim), device=dev)
        z = torch.zeros((1, w.kv_heads, w.head_dim), device=dev)
        flops = WL.hybrid_flops(w)
        qr, kr = V.vdit_rope_qk(qd, kd, grid)
        knorm = key_norm_bound(w.head_dim)  # the keys come out of the RMSNorm

        def step(i):
            V.vdit_attn_fwd(qr, kr, vd, mode="hybrid", chunk_tokens=w.chunk_tokens, state_s=s, state_z=z, workspace=ws,
                            overlap_tokens=w.overlap_tokens, key_norm_max=knorm, state_zero=True)
        form = "one call over the whole sequence from the zero state (delta + scan, chunk softmax + linear epilogue)"
    else:
        flops = WL.flops_full(w.tokens, w.tokens, w.heads, w.head_dim)

        def step(i):
            qr, kr = V.vdit_rope_qk(qd, kd, grid)
            V.vdit_attn_fwd(qr, kr, vd)
        form = "rope + full attention"
    wall, each, args.steps, args.warmup = _time_steps(step, args.steps, args.warmup)
    if w.mode == "rolling":
        stream()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(3)]
        for a, b in ev:
            a.record(); stream(); b.record()
        torch.cuda.synchronize()
        ms = sorted(a.elapsed_time(b) for a, b in ev)[1]
        sflops = sum(WL.flops_full(w.tokens, w.tokens * min(f + 1, w.n_slots), w.heads, w.head_dim)
                     for f in range(w.n_frames))
        extra["stream"] = {"frames": w.n_frames, "ms_median_of_3": round(ms, 3),
                           "ms_per_frame": round(ms / w.n_frames, 4), "TFLOPs": round(sflops / (ms * 1e-3) / 1e12, 1)}
    line = {"metric": METRIC, "value": round(flops / (wall * 1e-3) / 1e12, 2), "unit": "TFLOP/s",
            "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(wall, 4),
            "step_ms_median": round(each[len(each) // 2], 4), "step_ms_min": round(each[0], 4),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": w.dtype,
            "data": "synthetic (seeded N(0,1), bf16 RNE)",
            "config": {"workload": w.name, "mode": w.mode, "form": form, "tokens": w.tokens,
                       "heads": w.heads, "kv_heads": w.kv_heads, "head_dim": w.head_dim,
                       "kv_norm": w.kv_norm, "chunk_tokens": w.chunk_tokens,
                       "overlap_tokens": w.overlap_tokens, "reference_only": True},
            "pct_bf16_peak_step": round(100 * flops / (wall * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 2),
            "algorithmic_flops_per_step": flops}
    line.update(extra)
    return line


# -------------------------------------------------- profiler post-processing --

def calibrate_copy(nbytes: int = 1 << 30, reps: int = 5):
    """A plain device-to-device copy of known size, for scaling the HBM byte
    counters (FETCH_SIZE / WRITE_SIZE) of a profiler run: each launch reads and
    writes exactly nbytes."""
    import torch
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    src.fill_(1)
    torch.cuda.synchronize()
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibration": "copy", "bytes_read_per_launch": nbytes,
                      "bytes_written_per_launch": nbytes, "launches": reps}), flush=True)


def _csv_rows(run_dir: str, suffix: str):
    import csv
    import glob
    files = glob.glob(os.path.join(run_dir, "**", "*" + suffix), recursive=True)
    if not files:
        raise SystemExit(f"no *{suffix} under {run_dir}")
    rows = []
    for fn in files:
        with open(fn, newline="") as f:
            rows += list(csv.DictReader(f))
    return rows


def _counter_rows(run_dir: str):
    """(kernel name, counter name, value) rows of a rocprofv3 --pmc CSV run."""
    return [(r["Kernel_Name"], r["Counter_Name"], float(r["Counter_Value"]))
            for r in _csv_rows(run_dir, "counter_collection.csv")]


def _mean_counter(rows, kernel_substr: str, counter: str) -> tuple[float, int]:
    vals = [v for k, c, v in rows if kernel_substr in k and c == counter]
    if not vals:
        raise SystemExit(f"no {counter} rows for kernel matching {kernel_substr!r}")
    return sum(vals) / len(vals), len(vals)


def _copy_factors(run_root: str):
    nbytes = float(1 << 30)
    cf, _ = _mean_counter(_counter_rows(os.path.join(run_root, "cfetch")), "copyBuffer", "FETCH_SIZE")
    cw, _ = _mean_counter(_counter_rows(os.path.join(run_root, "cwrite")), "copyBuffer", "WRITE_SIZE")
    return nbytes, cf, cw, nbytes / (cf * 1024), nbytes / (cw * 1024)


def traffic_from(run_root: str, kernels=(("attn", "attn_mfma_kernel"), ("rope", "rope_qk_kernel")),
                 source: str = ATTN_SRC, total_of: str = "attn"):
    """Turn four rocprofv3 --pmc runs under run_root (fetch/, write/: the
    benchmark; cfetch/, cwrite/: `bench.py --calibrate-copy`) into HBM bytes per
    launch of each kernel.  FETCH_SIZE and WRITE_SIZE are in KiB per dispatch;
    each is scaled by the ratio (bytes actually copied) / (counter x 1024) of
    the 1 GiB copy."""
    nbytes, cf, cw, f_fetch, f_write = _copy_factors(run_root)
    out = {"kernel_source_sha256_16": src_hash(source), "calibration": {
        "copy_bytes": int(nbytes), "copy_FETCH_SIZE_KiB": cf, "copy_WRITE_SIZE_KiB": cw,
        "fetch_factor": round(f_fetch, 4), "write_factor": round(f_write, 4)}}
    for name, sub in kernels:
        fe, n_f = _mean_counter(_counter_rows(os.path.join(run_root, "fetch")), sub, "FETCH_SIZE")
        wr, n_w = _mean_counter(_counter_rows(os.path.join(run_root, "write")), sub, "WRITE_SIZE")
        out[name] = {"FETCH_SIZE_KiB": fe, "WRITE_SIZE_KiB": wr, "dispatches": [n_f, n_w],
                     "read_bytes": round(fe * 1024 * f_fetch), "write_bytes": round(wr * 1024 * f_write)}
    if total_of in out:
        out["hbm_bytes_per_launch"] = out[total_of]["read_bytes"] + out[total_of]["write_bytes"]
    return out


def hybrid_state_bytes(w) -> dict:
    """Algorithmic HBM bytes of the chunk-hybrid's linear-attention state
    kernels for workload w (bf16, B = 1), as the benchmark's step runs them
    (from the zero state, VDIT_ATTN_STATE_ZERO): the delta pass reads K and V
    of every token that enters the state (all but the last overlap_tokens,
    which the next call receives as context) and writes one float32 dS^T, dz
    per (chunk, token split, kv head); the scan reads those and writes S_c^T
    (bf16) and z_c (float32) per chunk and the outgoing state."""
    D, Hk, L = w.head_dim, w.kv_heads, w.tokens
    Ls = L - (w.overlap_tokens or 0)
    nch = -(-L // w.chunk_tokens)
    units = nch * Hk
    ns = max(1, min(8, -(-512 // units), w.chunk_tokens // 64))
    deltas = nch * ns * Hk * (D * D + D) * 4
    state = Hk * (D * D + D) * 4
    return {"delta": 2 * Ls * Hk * D * 2 + deltas,
            "scan": deltas + nch * Hk * (D * D * 2 + D * 4) + state,
            "token_splits": ns}


def kernel_stats_from(run_dir: str, workload: int, steps=None, warmup=None):
    """Per-kernel average durations of a rocprofv3 --kernel-trace --stats run of
    `bench.py --workload N` (run_kernel_stats.csv), with the algorithmic
    rates of the attention and linear-state kernels; for the decode and
    hybrid workloads, given the run's --steps and --warmup, also the
    averages over the timed steps' dispatches alone (run_kernel_trace.csv),
    from which the rates are then taken."""
    import workloads as WL
    w = WL.WORKLOADS[workload]
    rows = _csv_rows(run_dir, "kernel_stats.csv")
    out = {"workload": w.name, "kernels": {}}
    for r in rows:
        out["kernels"][r["Name"]] = {"calls": int(r["Calls"]), "avg_ns": float(r["AverageNs"]),
                                      "min_ns": float(r["MinNs"]), "max_ns": float(r["MaxNs"])}

    if w.mode in ("rolling", "hybrid") and steps and warmup is not None:
        # a decode or hybrid step launches each of its kernels once; the
        # setup (cache fill, input rotation) and the stream runs after the
        # timed pass use other kernel names or come later, so dispatches
        # [warmup, warmup + steps) of each kernel are the timed pass's
        per = {}
        for r in sorted(_csv_rows(run_dir, "kernel_trace.csv"), key=lambda r: int(r["Start_Timestamp"])):
            per.setdefault(r["Kernel_Name"], []).append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
        win = {}
        for name, d in per.items():
            if len(d) >= warmup + steps:
                t = d[warmup:warmup + steps]
                win[name] = {"dispatches": f"{warmup}..{warmup + steps - 1}", "avg_ns": round(sum(t) / len(t), 1),
                             "median_ns": sorted(t)[len(t) // 2]}
        out["timed_window"] = win
    win = out.get("timed_window", {})

    def avg(sub):
        v = [x["avg_ns"] for k, x in win.items() if sub in k] or \
            [x["avg_ns"] for k, x in out["kernels"].items() if sub in k]
        return v[0] if v else None
    if w.mode == "rolling":
        a = avg("attn_mfma_kernel")
        if a:
            out["attn_TFLOPs"] = round(WL.flops_full(w.tokens, w.tokens * w.n_slots, w.heads, w.head_dim)
                                       / a / 1e3, 1)
    if w.mode == "hybrid":
        b = hybrid_state_bytes(w)
        for name, sub in (("delta", "hybrid_delta"), ("scan", "hybrid_scan")):
            ns = avg(sub)
            if ns:
                out[name + "_GBps"] = round(b[name] / ns, 1)
                out[name + "_algorithmic_bytes"] = b[name]
        a = avg("attn_mfma_kernel")
        if a:
            out["attn_TFLOPs"] = round(WL.hybrid_flops(w) / a / 1e3, 1)
    return out


# --------------------------------------------------------------------- main --

def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed steps (default: 50 on the 32760-token layer; on the other workloads "
                         "as many as fill 100 ms, at least 50)")
    ap.add_argument("--warmup", type=int, default=None,
                    help="untimed steps first (default: 10 on the 32760-token layer; on the other "
                         "workloads as many as fill 100 ms, at least 10)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=32760,
                    help="query rows of the oracle's timed sample (full: all rows at the default; ring: at most 4096)")
    ap.add_argument("--workload", type=int, default=2)
    ap.add_argument("--no-peaks", action="store_true",
                    help="skip the RoPE-over-rotated-buffers and reference-peak measurements (profiler passes)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run only a 1 GiB device copy (HBM counter calibration)")
    ap.add_argument("--traffic-from", metavar="DIR",
                    help="summarise rocprofv3 --pmc runs DIR/{fetch,write,cfetch,cwrite} "
                         "into the traffic JSON (no GPU needed)")
    ap.add_argument("--kernel-stats-from", metavar="DIR",
                    help="summarise a rocprofv3 --kernel-trace --stats run of --workload N (no GPU needed)")
    args = ap.parse_args()
    if args.traffic_from:
        t = traffic_from(args.traffic_from)
        os.makedirs(os.path.dirname(TRAFFIC_FILE), exist_ok=True)
        with open(TRAFFIC_FILE, "w") as f:
            json.dump(t, f, indent=1)
            f.write("\n")
        print(json.dumps(t), flush=True)
        return
    if args.kernel_stats_from:
        print(json.dumps(kernel_stats_from(args.kernel_stats_from, args.workload, args.steps, args.warmup)),
              flush=True)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(the layer's sharding is described in the design notes). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    if args.calibrate_copy:
        calibrate_copy()
        return
    import workloads as WL
    w = WL.WORKLOADS[args.workload]
    base = None if args.no_cpu_baseline or w.mode == "full" and w.dtype != "bf16" else \
        cpu_baseline(w, args.cpu_rows)
    if args.workload == 2:
        args.steps = 50 if args.steps is None else args.steps
        args.warmup = 10 if args.warmup is None else args.warmup
    out = bench_full(args) if args.workload == 2 else bench_other(args)
    out["cpu_baseline"] = base
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
