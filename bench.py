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
`cpu_baseline` times the fp64 oracle on a bounded sample of query rows.

  python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu-baseline]
  python bench.py --workload N   (other workloads, for reference; one JSON line each)
"""
from __future__ import annotations

import argparse
import math
import hashlib
import json
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


def cpu_baseline(w, n_rows: int, seed: int = 99):
    """fp64 oracle on a bounded sample: rope over the whole grid (every key needs
    it) plus attention of n_rows sampled query rows x all heads against all keys."""
    import numpy as np
    import oracle as O
    import workloads as WL
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:  # pragma: no cover
        threads = 1
    q, k, v = WL.workload_inputs(w)
    rows = WL.sample_rows(w.tokens, n_rows, seed)
    t0 = time.perf_counter()
    wq, wk = O.rope_qk(q.values, k.values, w.grid, w.pairs)
    O.attention(wq[:, rows], wk, v.values)
    dt = time.perf_counter() - t0
    flops = WL.flops_full(len(rows), w.tokens, w.heads, w.head_dim)
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{len(rows)} of {w.tokens} query rows x {w.heads} heads vs all {w.tokens} keys, "
                      f"plus RMSNorm+RoPE of all tokens; {dt:.1f} s wall",
            "seconds": dt}


def bench_full(args):
    import numpy as np
    import torch
    import video_diffusion_transformer_rmsnorm_amd as V
    import workloads as WL

    w = WL.WORKLOADS[2]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    q, k, v = WL.workload_inputs(w)

    def up(t):
        return torch.from_numpy(np.ascontiguousarray(t.bits).view(np.int16)).view(torch.bfloat16).to(dev)

    qd, kd, vd = up(q), up(k), up(v)
    del q, k, v
    qr, kr = torch.empty_like(qd), torch.empty_like(kd)
    o = torch.empty_like(qd)
    lse = torch.empty((1, w.heads, w.tokens), dtype=torch.float32, device=dev)
    grid = V.make_grid(*w.grid, w.pairs)
    stream = torch.cuda.current_stream()

    # the step's keys come out of vdit_rope_qk RMS-normalised (gain 1): their
    # norms are at most sqrt(D) up to bf16 rounding, which lets the attention
    # call skip its own pass over the keys (same results, see vdit.h)
    knorm = key_norm_bound(w.head_dim)

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        V.vdit_rope_qk(qd, kd, grid, q_out=qr, k_out=kr)
        if ev is not None:
            ev[1].record(stream)
        V.vdit_attn_fwd(qr, kr, vd, o=o, lse=lse, key_norm_max=knorm)
        if ev is not None:
            ev[2].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    rope_each = [e[0].elapsed_time(e[1]) for e in evs]
    attn_each = sorted(e[1].elapsed_time(e[2]) for e in evs)
    rope_ms = sum(rope_each) / args.steps
    attn_ms = sum(attn_each) / args.steps
    ms_step = wall * 1e3 / args.steps
    flops = WL.flops_full(w.tokens, w.tokens, w.heads, w.head_dim)
    rope_bytes = 2 * 2 * w.tokens * w.heads * w.head_dim * 2  # q,k read + write, bf16
    achieved = flops / (attn_ms * 1e-3) / 1e12
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
                     "traffic": measured_traffic(), "kernel": "attn_mfma_kernel<128,8,1>",
                     "algorithmic_flops_per_launch": flops},
    }
    out["measured_peaks"] = measured_peaks(achieved, out["rope_GBps"])
    return out, w


def measured_peaks(attn_tflops: float, rope_gbps: float, reps: int = 10):
    """Reference rates measured on the same device after the timed region: a
    bf16 library GEMM (8192^3, hipBLASLt) as the sustained dense-MFMA rate and
    a 1 GiB device-to-device copy as the sustained HBM rate, with the
    attention and RoPE rates as fractions of them (context for the nominal
    peaks in `roofline`, not a replacement)."""
    import torch
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
    return {"gemm_bf16_8192_TFLOPs": round(gemm, 1), "attn_frac_of_gemm": round(attn_tflops / gemm, 4),
            "copy_1GiB_GBps": round(copy, 1), "rope_frac_of_copy": round(rope_gbps / copy, 4)}


def key_norm_bound(head_dim: int) -> float:
    """Bound on the norm of keys RMS-normalised with gain 1 and stored in
    bf16: sqrt(head_dim), widened for the rounding of each element."""
    return math.sqrt(head_dim) * (1.0 + 2.0 ** -7)


def bench_other(args):
    """Reference timings of the other workloads (not the headline line)."""
    import numpy as np
    import torch
    import video_diffusion_transformer_rmsnorm_amd as V
    import workloads as WL

    w = WL.WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    q, k, v = WL.workload_inputs(w)

    def up(t):
        if t.dtype == "bf16":
            return torch.from_numpy(np.ascontiguousarray(t.bits).view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(t.values.astype(np.float32)).to(dev)

    qd, kd, vd = up(q), up(k), up(v)
    grid = V.make_grid(*w.grid, w.pairs)
    if w.mode == "ring":
        q0, nq = w.q_range
        qq = qd[:, q0:q0 + nq].contiguous()
        kcs = [kd[:, s:s + n].contiguous() for s, n in w.kv_chunks]
        vcs = [vd[:, s:s + n].contiguous() for s, n in w.kv_chunks]
        flops = sum(WL.flops_full(nq, n, w.heads, w.head_dim) for _, n in w.kv_chunks)

        def step():
            V.vdit_attn_fwd(qq, mode="ring", k_chunks=kcs, v_chunks=vcs)
    elif w.mode == "rolling":
        kc = torch.zeros((1, w.n_slots, w.tokens, w.kv_heads, w.head_dim), dtype=qd.dtype, device=dev)
        vc = torch.zeros_like(kc)
        for f in range(w.n_slots):
            # the cache starts full of normalised, rotated keys, as the steps leave it
            V.vdit_rope_qk(None, kd[f:f + 1], grid, k_out=kc[:, f])
            vc[:, f].copy_(vd[f:f + 1])
        flops = WL.flops_full(w.tokens, w.tokens * w.n_slots, w.heads, w.head_dim)
        frame = [w.n_slots]
        t_step = w.grid[0]
        q_norm = False if w.kv_norm else None

        def step():
            # one decode step: rotate q (KV-norm: without its norm), normalise and
            # rotate k straight into the cache slot, values into their slot
            # (normalised under KV-norm), then attend over the window
            f = frame[0]
            i, slot = f % w.n_frames, f % w.n_slots
            qi = qd[i:i + 1]
            V.vdit_rope_qk(qi, kd[i:i + 1], grid, q_out=qi, k_out=kc[:, slot], t_offset=t_step * f,
                           q_norm=q_norm)
            if w.kv_norm:
                V.vdit_rms_norm(vd[i:i + 1], out=vc[:, slot])
            else:
                vc[:, slot].copy_(vd[i:i + 1])
            V.vdit_attn_fwd(qi, mode="rolling", k_cache=kc, v_cache=vc, frame=f,
                            key_norm_max=key_norm_bound(w.head_dim))
            frame[0] += 1
    elif w.mode == "hybrid":
        s = torch.zeros((1, w.kv_heads, w.head_dim, w.head_dim), device=dev)
        z = torch.zeros((1, w.kv_heads, w.head_dim), device=dev)
        flops = WL.hybrid_flops(w)

        def step():
            s.zero_(); z.zero_()
            V.vdit_attn_fwd(qd, kd, vd, mode="hybrid", chunk_tokens=w.chunk_tokens, state_s=s, state_z=z,
                            overlap_tokens=w.overlap_tokens)
    else:
        flops = WL.flops_full(w.tokens, w.tokens, w.heads, w.head_dim)

        def step():
            V.vdit_rope_qk(qd, kd, grid)
            V.vdit_attn_fwd(qd, kd, vd)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    t0 = time.perf_counter()
    for e in evs:
        e[0].record()
        step()
        e[1].record()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / args.steps
    each = sorted(a.elapsed_time(b) for a, b in evs)
    return {"metric": METRIC, "value": round(flops / (ms * 1e-3) / 1e12, 2), "unit": "TFLOP/s",
            "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
            "step_ms_median": round(each[len(each) // 2], 4), "step_ms_min": round(each[0], 4),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": w.dtype,
            "data": "synthetic", "config": {"workload": w.name, "mode": w.mode, "tokens": w.tokens,
                                            "heads": w.heads, "kv_heads": w.kv_heads, "head_dim": w.head_dim,
                                            "kv_norm": w.kv_norm, "chunk_tokens": w.chunk_tokens,
                                            "overlap_tokens": w.overlap_tokens, "reference_only": True}}


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


def _counter_rows(run_dir: str):
    """(kernel name, counter name, value) rows of a rocprofv3 --pmc CSV run."""
    import csv
    import glob
    files = glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no *counter_collection.csv under {run_dir}")
    rows = []
    for fn in files:
        with open(fn, newline="") as f:
            for r in csv.DictReader(f):
                rows.append((r["Kernel_Name"], r["Counter_Name"], float(r["Counter_Value"])))
    return rows


def _mean_counter(rows, kernel_substr: str, counter: str) -> tuple[float, int]:
    vals = [v for k, c, v in rows if kernel_substr in k and c == counter]
    if not vals:
        raise SystemExit(f"no {counter} rows for kernel matching {kernel_substr!r}")
    return sum(vals) / len(vals), len(vals)


def traffic_from(run_root: str):
    """Turn four rocprofv3 --pmc runs under run_root (fetch/, write/: this bench;
    cfetch/, cwrite/: `bench.py --calibrate-copy`) into HBM bytes per attention
    launch.  FETCH_SIZE and WRITE_SIZE are in KiB per dispatch; each is scaled by
    the ratio (bytes actually copied) / (counter x 1024) of the 1 GiB copy."""
    nbytes = float(1 << 30)
    cf, _ = _mean_counter(_counter_rows(os.path.join(run_root, "cfetch")), "copyBuffer", "FETCH_SIZE")
    cw, _ = _mean_counter(_counter_rows(os.path.join(run_root, "cwrite")), "copyBuffer", "WRITE_SIZE")
    f_fetch, f_write = nbytes / (cf * 1024), nbytes / (cw * 1024)
    out = {"kernel_source_sha256_16": src_hash(ATTN_SRC), "calibration": {
        "copy_bytes": int(nbytes), "copy_FETCH_SIZE_KiB": cf, "copy_WRITE_SIZE_KiB": cw,
        "fetch_factor": round(f_fetch, 4), "write_factor": round(f_write, 4)}}
    for name, sub in (("attn", "attn_mfma_kernel"), ("rope", "rope_qk_kernel")):
        fe, n_f = _mean_counter(_counter_rows(os.path.join(run_root, "fetch")), sub, "FETCH_SIZE")
        wr, n_w = _mean_counter(_counter_rows(os.path.join(run_root, "write")), sub, "WRITE_SIZE")
        out[name] = {"FETCH_SIZE_KiB": fe, "WRITE_SIZE_KiB": wr, "dispatches": [n_f, n_w],
                     "read_bytes": round(fe * 1024 * f_fetch), "write_bytes": round(wr * 1024 * f_write)}
    out["hbm_bytes_per_launch"] = out["attn"]["read_bytes"] + out["attn"]["write_bytes"]
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=8192,
                    help="query rows of the oracle's timed sample")
    ap.add_argument("--workload", type=int, default=2)
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run only a 1 GiB device copy (HBM counter calibration)")
    ap.add_argument("--traffic-from", metavar="DIR",
                    help="summarise rocprofv3 --pmc runs DIR/{fetch,write,cfetch,cwrite} "
                         "into the traffic JSON (no GPU needed)")
    args = ap.parse_args()
    if args.traffic_from:
        t = traffic_from(args.traffic_from)
        os.makedirs(os.path.dirname(TRAFFIC_FILE), exist_ok=True)
        with open(TRAFFIC_FILE, "w") as f:
            json.dump(t, f, indent=1)
            f.write("\n")
        print(json.dumps(t), flush=True)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(the layer's sharding is described in the design notes). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    if args.calibrate_copy:
        calibrate_copy()
        return
    if args.workload != 2:
        print(json.dumps(bench_other(args)), flush=True)
        return
    out, w = bench_full(args)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, args.cpu_rows)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
