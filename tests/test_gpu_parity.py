"""GPU parity: the HIP path through the C ABI against the fp64 oracle.

Inputs come from the seeded generators in ``workloads``; expected values from
``oracle`` only.  Small cases span several tiles and ragged tails; the
full-size workloads are checked on seeded samples of query rows (each row
against every key) in the launch configuration the benchmark times.
"""
import math
import os
import subprocess

import numpy as np
import pytest
import torch

import oracle as O
import video_diffusion_transformer_rmsnorm_amd as V
import workloads as WL
from parity import check, check_lse, from_dev, log, to_dev

pytestmark = pytest.mark.gpu


def raw(shape, seed, dtype):
    rng = np.random.default_rng(seed)
    return WL.draw(shape, rng, dtype)


def ws(dtype):
    return "bf16" if dtype == torch.bfloat16 else "f32"


# --------------------------------------------------------------------- rope --

@pytest.mark.parametrize("dtype,D,pairs", [("bf16", 128, (22, 21, 21)), ("bf16", 64, (12, 10, 10)),
                                           ("f32", 64, (12, 10, 10)), ("f32", 128, (20, 22, 22))])
def test_rope_small_ragged(dtype, D, pairs):
    grid = (3, 5, 7)
    B, L, Hq, Hk = 2, 97, 3, 1
    log(f"rope small {dtype} D={D} pairs={pairs} B={B} L={L}")
    q = raw((B, L, Hq, D), 11, dtype); k = raw((B, L, Hk, D), 12, dtype)
    qd, kd = to_dev(q), to_dev(k)
    g = V.make_grid(*grid, pairs)
    qo, ko = V.vdit_rope_qk(qd, kd, g, token0=5, t_offset=3)
    torch.cuda.synchronize()
    wq, wk = O.rope_qk(q.values, k.values, grid, pairs, token0=5, t_offset=3)
    check(qo, wq, dtype, "q"); check(ko, wk, dtype, "k")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_rope_inplace_gain_nonorm_large_offset(dtype):
    D, pairs, grid = 64, (12, 10, 10), (1, 34, 60)
    L = 2040
    log(f"rope in-place / gains / no-norm / t_offset {dtype}")
    q = raw((1, L, 4, D), 21, dtype); k = raw((1, L, 2, D), 22, dtype)
    rng = np.random.default_rng(23)
    qg = (1.0 + 0.1 * rng.standard_normal(D)).astype(np.float32)
    kg = (1.0 + 0.1 * rng.standard_normal(D)).astype(np.float32)
    qd, kd = to_dev(q), to_dev(k)
    g = V.make_grid(*grid, pairs)
    V.vdit_rope_qk(qd, kd, g, q_out=qd, k_out=kd, t_offset=100003,
                   q_gain=torch.from_numpy(qg).cuda(), k_gain=torch.from_numpy(kg).cuda())
    torch.cuda.synchronize()
    wq, wk = O.rope_qk(q.values, k.values, grid, pairs, t_offset=100003, q_gain=qg, k_gain=kg)
    check(qd, wq, dtype, "q in place"); check(kd, wk, dtype, "k in place")
    qo, _ = V.vdit_rope_qk(to_dev(q), None, g, norm=False)
    torch.cuda.synchronize()
    wq2, _ = O.rope_qk(q.values, k.values, grid, pairs, norm=False)
    check(qo, wq2, dtype, "q no-norm")


@pytest.mark.parametrize("dtype,D", [("bf16", 64), ("bf16", 128), ("f32", 64), ("f32", 128)])
def test_rms_norm_values_ragged_inplace_gain(dtype, D):
    # per-head RMSNorm alone (the values of KV-norm attention): out of place,
    # in place, with a gain; row count not a multiple of the block's rows
    B, L, H = 2, 333, 3
    log(f"rms norm {dtype} D={D} B={B} L={L} H={H}")
    vals = raw((B, L, H, D), 31, dtype).values
    vals[0, 5] *= 40.0  # a few large rows, rounded again to the element type below
    v32 = vals.astype(np.float32)
    if dtype == "bf16":
        bits = WL.f32_to_bf16_bits(v32)
        x = WL.Tensor(WL.bf16_bits_to_f64(bits), bits, dtype)
    else:
        x = WL.Tensor(v32.astype(np.float64), None, dtype)
    g = (1.0 + 0.1 * np.random.default_rng(32).standard_normal(D)).astype(np.float32)
    xd = to_dev(x)
    out = V.vdit_rms_norm(xd)
    torch.cuda.synchronize()
    check(out, O.rmsnorm(x.values), dtype, "rms norm")
    V.vdit_rms_norm(xd, out=xd, gain=torch.from_numpy(g).cuda(), eps=1e-5)
    torch.cuda.synchronize()
    check(xd, O.rmsnorm(x.values, 1e-5, g), dtype, "rms norm in place with gain")
    empty = torch.empty((1, 0, H, D), dtype=xd.dtype, device="cuda")
    V.vdit_rms_norm(empty, out=empty)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_rope_without_query_norm(dtype):
    # KV-norm: keys normalised then rotated, queries rotated only
    D, pairs, grid = 64, (12, 10, 10), (4, 9, 10)
    L = 360
    log(f"rope with k norm only {dtype}")
    q = raw((1, L, 8, D), 33, dtype); k = raw((1, L, 1, D), 34, dtype)
    qo, ko = V.vdit_rope_qk(to_dev(q), to_dev(k), V.make_grid(*grid, pairs), t_offset=7, q_norm=False)
    torch.cuda.synchronize()
    wq, wk = O.rope_qk(q.values, k.values, grid, pairs, t_offset=7, q_norm=False)
    check(qo, wq, dtype, "q rotated only"); check(ko, wk, dtype, "k normalised and rotated")


@pytest.mark.parametrize("dtype,D,pairs", [("bf16", 64, (12, 10, 10)), ("bf16", 128, (22, 21, 21)),
                                           ("f32", 64, (12, 10, 10))])
def test_rope_qkv_values_in_the_same_launch(dtype, D, pairs):
    """vdit_rope_qkv: q and k as vdit_rope_qk gives them and the values
    copied, or normalised as vdit_rms_norm gives them (the same bits), also
    written straight into a rolling-cache slot and in place; ragged token
    count, grouped-query heads, gains; q, k, v against the oracle."""
    grid = (4, 9, 10)
    B, L, Hq, Hk = 2, 337, 6, 2
    log(f"rope qkv {dtype} D={D} B={B} L={L} Hq={Hq} Hk={Hk}")
    q = raw((B, L, Hq, D), 41, dtype); k = raw((B, L, Hk, D), 42, dtype); v = raw((B, L, Hk, D), 43, dtype)
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    g = V.make_grid(*grid, pairs)
    gv = (1.0 + 0.1 * np.random.default_rng(44).standard_normal(D)).astype(np.float32)
    gk = (1.0 + 0.1 * np.random.default_rng(45).standard_normal(D)).astype(np.float32)
    gvd, gkd = torch.from_numpy(gv).cuda(), torch.from_numpy(gk).cuda()
    # values copied: q and k exactly as vdit_rope_qk
    q1, k1, v1 = V.vdit_rope_qkv(qd, kd, vd, g, token0=11, t_offset=5, k_gain=gkd)
    q2, k2 = V.vdit_rope_qk(qd, kd, g, token0=11, t_offset=5, k_gain=gkd)
    # KV-norm: q rotated only, k normalised and rotated, values normalised
    q3, k3, v3 = V.vdit_rope_qkv(qd, kd, vd, g, token0=11, t_offset=5, q_norm=False, v_norm=True, v_gain=gvd)
    q4, k4 = V.vdit_rope_qk(qd, kd, g, token0=11, t_offset=5, q_norm=False)
    v4 = V.vdit_rms_norm(vd, gain=gvd)
    torch.cuda.synchronize()
    assert torch.equal(q1, q2) and torch.equal(k1, k2), "q, k differ from vdit_rope_qk"
    assert torch.equal(v1, vd), "copied values differ"
    assert torch.equal(q3, q4) and torch.equal(k3, k4), "q, k differ from vdit_rope_qk (KV-norm)"
    assert torch.equal(v3, v4), "normalised values differ from vdit_rms_norm"
    wq, wk = O.rope_qk(q.values, k.values, grid, pairs, token0=11, t_offset=5, q_norm=False)
    check(q3, wq, dtype, "q rotated only"); check(k3, wk, dtype, "k normalised and rotated")
    check(v3, O.rmsnorm(v.values, 1e-6, gv), dtype, "v normalised with gain")
    # a decode frame's two cache slots (B = 1), and values in place
    kc = torch.zeros((1, 3, L, Hk, D), dtype=kd.dtype, device="cuda"); vc = torch.zeros_like(kc)
    qo = torch.empty_like(qd[:1])
    V.vdit_rope_qkv(qd[:1], kd[:1], vd[:1], g, q_out=qo, k_out=kc[:, 2], v_out=vc[:, 2], v_norm=True)
    vin = vd[1:].clone()
    V.vdit_rope_qkv(None, None, vin, g, v_out=vin, v_norm=True)
    torch.cuda.synchronize()
    assert torch.equal(kc[:, 2], V.vdit_rope_qk(None, kd[:1], g)[1]), "k in the slot"
    assert torch.equal(vc[:, 2], V.vdit_rms_norm(vd[:1])), "v in the slot"
    assert torch.equal(vc[:, :2], torch.zeros_like(vc[:, :2])) and torch.equal(kc[:, :2], torch.zeros_like(kc[:, :2]))
    assert torch.equal(vin, V.vdit_rms_norm(vd[1:])), "v normalised in place"


def test_rope_full_size_wan13b():
    w = WL.WORKLOADS[2]
    log("rope full size 32760 x 12 x 128 bf16")
    q, k, _ = WL.workload_inputs(w)
    qo, ko = V.vdit_rope_qk(to_dev(q), to_dev(k), V.make_grid(*w.grid, w.pairs))
    torch.cuda.synchronize()
    wq, wk = O.rope_qk(q.values, k.values, w.grid, w.pairs)
    check(qo, wq, "bf16", "q"); check(ko, wk, "bf16", "k")


# --------------------------------------------------------------- attention --

@pytest.mark.parametrize("dtype,D,Lq,Lkv,Hq,Hk", [
    ("bf16", 128, 300, 333, 4, 2), ("bf16", 64, 300, 333, 4, 4), ("bf16", 128, 1, 77, 2, 1),
    ("bf16", 64, 513, 64, 2, 2), ("bf16", 128, 700, 1, 2, 2),
    ("f32", 64, 130, 97, 2, 1), ("f32", 128, 65, 200, 2, 2),
])
def test_full_attention_small(dtype, D, Lq, Lkv, Hq, Hk):
    log(f"full attention {dtype} D={D} Lq={Lq} Lkv={Lkv} Hq={Hq} Hk={Hk}")
    q = raw((2, Lq, Hq, D), 31, dtype); k = raw((2, Lkv, Hk, D), 32, dtype); v = raw((2, Lkv, Hk, D), 33, dtype)
    o, lse = V.vdit_attn_fwd(to_dev(q), to_dev(k), to_dev(v))
    torch.cuda.synchronize()
    wo, wl = O.attention(q.values, k.values, v.values)
    check(o, wo, dtype, "O"); check_lse(lse, wl, dtype, "LSE")


def test_full_attention_empty_keys_and_scale():
    log("full attention: no keys; explicit scale")
    q = raw((1, 40, 2, 64), 41, "bf16")
    kd = torch.empty((1, 0, 2, 64), dtype=torch.bfloat16, device="cuda")
    o, lse = V.vdit_attn_fwd(to_dev(q), kd, kd)
    torch.cuda.synchronize()
    assert (from_dev(o) == 0).all() and np.isneginf(from_dev(lse)).all()
    k = raw((1, 90, 2, 64), 42, "bf16"); v = raw((1, 90, 2, 64), 43, "bf16")
    o, lse = V.vdit_attn_fwd(to_dev(q), to_dev(k), to_dev(v), scale=0.3)
    torch.cuda.synchronize()
    wo, wl = O.attention(q.values, k.values, v.values, 0.3)
    check(o, wo, "bf16", "O scale 0.3"); check_lse(lse, wl, "bf16", "LSE scale 0.3")


@pytest.mark.parametrize("norm", [True, False])
def test_tiny_workload_f32_end_to_end(norm):
    w = WL.WORKLOADS[1]
    log(f"tiny fp32 workload 72 tokens, norm={norm}")
    q, k, v = WL.workload_inputs(w)
    g = V.make_grid(*w.grid, w.pairs)
    qr, kr = V.vdit_rope_qk(to_dev(q), to_dev(k), g, norm=norm)
    o, lse = V.vdit_attn_fwd(qr, kr, to_dev(v), scale=1.0 / 8)
    torch.cuda.synchronize()
    wq, wk = O.rope_qk(q.values, k.values, w.grid, w.pairs, norm=norm)
    wo, wl = O.attention(wq, wk, v.values, 1.0 / 8)
    check(qr, wq, "f32", "q roped"); check(o, wo, "f32", "O"); check_lse(lse, wl, "f32", "LSE")


@pytest.mark.parametrize("D", [128, 64])
def test_full_attention_wide_workgroups_sampled(D):
    # 8 query heads x ceil(16347 / 256) = 512 workgroups of 256 queries: two
    # even rounds on a 256-CU part, so the 8-wavefront workgroup shape runs;
    # ragged query and key tails, grouped-query heads.
    Lq, Lkv, Hq, Hk = 16347, 5013, 8, 2
    log(f"full attention, 256-query workgroups: D={D} Lq={Lq} Lkv={Lkv} Hq={Hq} Hk={Hk}")
    q = raw((1, Lq, Hq, D), 61, "bf16"); k = raw((1, Lkv, Hk, D), 62, "bf16"); v = raw((1, Lkv, Hk, D), 63, "bf16")
    o, lse = V.vdit_attn_fwd(to_dev(q), to_dev(k), to_dev(v))
    torch.cuda.synchronize()
    rows = WL.sample_rows(Lq, 160, seed=64)
    rows = np.unique(np.concatenate([rows, [0, 31, 32, 255, 256, 16127, 16128, Lq - 1]]))
    wo, wl = O.attention(q.values[:, rows], k.values, v.values)
    check(from_dev(o)[:, rows], wo, "bf16", "O (sampled rows)")
    check_lse(from_dev(lse)[:, :, rows], wl, "bf16", "LSE (sampled rows)")


@pytest.mark.parametrize("D", [128, 64])
def test_full_attention_key_split(D):
    # 16 workgroups of 128 queries: the keys are cut into 8 ranges of 640
    # (the last one ragged) whose float32 partials are merged; with a
    # workspace too small for the partials the same call runs unsplit.
    Lq, Lkv, Hq, Hk = 1000, 5000, 2, 1
    log(f"full attention with key split: D={D} Lq={Lq} Lkv={Lkv} Hq={Hq} Hk={Hk}")
    q = raw((1, Lq, Hq, D), 71, "bf16"); k = raw((1, Lkv, Hk, D), 72, "bf16"); v = raw((1, Lkv, Hk, D), 73, "bf16")
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    o_split, lse_split = V.vdit_attn_fwd(qd, kd, vd)
    o_plain, lse_plain = V.vdit_attn_fwd(qd, kd, vd, workspace=torch.empty(256, dtype=torch.uint8, device="cuda"))
    torch.cuda.synchronize()
    wo, wl = O.attention(q.values, k.values, v.values)
    check(o_split, wo, "bf16", "O (split)"); check_lse(lse_split, wl, "bf16", "LSE (split)")
    check(o_plain, wo, "bf16", "O (unsplit)"); check_lse(lse_plain, wl, "bf16", "LSE (unsplit)")


@pytest.mark.parametrize("D", [128, 64])
def test_full_attention_key_split_two_ranges(D):
    """12 workgroups of 128 queries (GQA, 4 query heads on 2 KV heads) split
    the keys into two ranges, [0, 320) and [320, 513): the second ends a
    whole tile before the first.  The computed key-norm bound, the caller's
    bound (RMS-normalised keys; the same bits as the computed one) and a
    workspace too small for bound and partials (online maximum, unsplit) all
    match the oracle."""
    Lq, Lkv, Hq, Hk = 300, 513, 4, 2
    log(f"full attention, key split in two ranges: D={D} Lq={Lq} Lkv={Lkv} Hq={Hq} Hk={Hk}")
    q = raw((1, Lq, Hq, D), 191, "bf16"); k = raw((1, Lkv, Hk, D), 192, "bf16"); v = raw((1, Lkv, Hk, D), 193, "bf16")
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    wo, wl = O.attention(q.values, k.values, v.values)
    o1, l1 = V.vdit_attn_fwd(qd, kd, vd)
    o2, l2 = V.vdit_attn_fwd(qd, kd, vd, workspace=torch.empty(16, dtype=torch.uint8, device="cuda"))
    torch.cuda.synchronize()
    check(o1, wo, "bf16", "O (computed bound)"); check_lse(l1, wl, "bf16", "LSE (computed bound)")
    check(o2, wo, "bf16", "O (online maximum, unsplit)"); check_lse(l2, wl, "bf16", "LSE (online maximum, unsplit)")
    # RMS-normalised keys under the caller's bound
    pairs = (22, 21, 21) if D == 128 else (12, 10, 10)
    qr = V.vdit_rope_qk(qd, None, V.make_grid(1, 1, Lq, pairs))[0]
    kr2 = V.vdit_rope_qk(None, kd, V.make_grid(1, 1, Lkv, pairs))[1]
    o3, l3 = V.vdit_attn_fwd(qr, kr2, vd, key_norm_max=math.sqrt(D) * (1 + 2 ** -7))
    o4, l4 = V.vdit_attn_fwd(qr, kr2, vd)
    torch.cuda.synchronize()
    assert torch.equal(o3, o4) and torch.equal(l3, l4), "caller's bound and computed bound differ"
    wo, wl = O.attention(from_dev(qr), from_dev(kr2), v.values)
    check(o3, wo, "bf16", "O (caller's bound)"); check_lse(l3, wl, "bf16", "LSE (caller's bound)")


@pytest.mark.parametrize("D,Lq", [(128, 16347), (64, 16347), (128, 9001), (64, 9001)])
def test_full_attention_bounded_and_online_softmax(D, Lq):
    # Lq 16347: 256-query workgroups (8 heads x 64 query tiles: two even
    # rounds on 256 CUs); Lq 9001: 128-query workgroups (8 heads x 71 tiles,
    # no key split).  Both use the key-norm bound: a wavefront whose queries
    # satisfy 2 c2 |q| max|k| <= 64 skips the running maximum.  Query rows
    # 4000..6099 are scaled by 8, beyond that bound, so wavefronts of both
    # kinds share workgroups.  Without the bound (workspace too small) every
    # wavefront keeps the online maximum.
    Lkv, Hq, Hk = 3001, 8, 2
    log(f"bounded-score and online-max softmax: D={D} Lq={Lq} Lkv={Lkv} Hq={Hq} Hk={Hk}")
    rng = np.random.default_rng(81)
    q64 = rng.standard_normal((1, Lq, Hq, D))
    q64[:, 4000:6100] *= 8.0
    k64 = rng.standard_normal((1, Lkv, Hk, D)); v64 = rng.standard_normal((1, Lkv, Hk, D))

    def bf16(x64):
        bits = WL.f32_to_bf16_bits(x64.astype(np.float32))
        return WL.Tensor(WL.bf16_bits_to_f64(bits), bits, "bf16")
    q, k, v = bf16(q64), bf16(k64), bf16(v64)
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    o_b, lse_b = V.vdit_attn_fwd(qd, kd, vd)
    o_o, lse_o = V.vdit_attn_fwd(qd, kd, vd, workspace=torch.empty(16, dtype=torch.uint8, device="cuda"))
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([WL.sample_rows(Lq, 128, seed=82), np.arange(3990, 4010),
                                     np.arange(6090, 6110), [0, Lq - 1]]))
    wo, wl = O.attention(q.values[:, rows], k.values, v.values)
    for o, lse, tag in ((o_b, lse_b, "bounded"), (o_o, lse_o, "online")):
        check(from_dev(o)[:, rows], wo, "bf16", f"O ({tag}, sampled rows)")
        check_lse(from_dev(lse)[:, :, rows], wl, "bf16", f"LSE ({tag}, sampled rows)")


def test_d64_workgroups_sized_for_three_per_cu():
    """D = 64, 32 query heads on 8 KV heads x ceil(2500 / 128) = 640
    workgroups of 128 queries: more than one round at two per CU on a
    256-CU part but one round at three, so the instance whose registers are
    sized for three wavefronts per SIMD runs.  Ragged query and key tails;
    query rows 1000..1299 scaled by 8 so that wavefronts with and without
    the bounded-score path share workgroups; every row against the oracle,
    with the computed key bound and with the online maximum alone."""
    D, Lq, Lkv, Hq, Hk = 64, 2500, 700, 32, 8
    log(f"D=64 call of one round at three workgroups per CU: Lq={Lq} Lkv={Lkv} Hq={Hq} Hk={Hk}")
    rng = np.random.default_rng(91)
    q64 = rng.standard_normal((1, Lq, Hq, D))
    q64[:, 1000:1300] *= 8.0
    k64 = rng.standard_normal((1, Lkv, Hk, D)); v64 = rng.standard_normal((1, Lkv, Hk, D))

    def bf16(x64):
        bits = WL.f32_to_bf16_bits(x64.astype(np.float32))
        return WL.Tensor(WL.bf16_bits_to_f64(bits), bits, "bf16")
    q, k, v = bf16(q64), bf16(k64), bf16(v64)
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    o_b, lse_b = V.vdit_attn_fwd(qd, kd, vd)
    o_o, lse_o = V.vdit_attn_fwd(qd, kd, vd, workspace=torch.empty(16, dtype=torch.uint8, device="cuda"))
    torch.cuda.synchronize()
    wo, wl = O.attention(q.values, k.values, v.values)
    for o, lse, tag in ((o_b, lse_b, "bounded"), (o_o, lse_o, "online")):
        check(o, wo, "bf16", f"O ({tag})")
        check_lse(lse, wl, "bf16", f"LSE ({tag})")


@pytest.mark.parametrize("D", [128, 64])
def test_caller_key_norm_bound(D):
    """key_norm_max replaces the key-norm pass.  Keys RMS-normalised and
    rotated by vdit_rope_qk have |k| <= sqrt(D) (1 + 2^-7); with that bound
    every wavefront takes the same path as with the computed one, so FULL,
    RING (one launch) and ROLLING give the same bits.  A bound far above the
    keys' norms sends every wavefront to the online maximum: checked against
    the oracle."""
    L, H = 9001, 16
    pairs = (22, 21, 21) if D == 128 else (12, 10, 10)
    grid = (9, 31, 33)
    log(f"caller key-norm bound: D={D} L={L} H={H}")
    q, k, v = WL.draw_qkv((1, L, H, D), (1, L, H, D), 91, "bf16")
    qr, kr = V.vdit_rope_qk(to_dev(q), to_dev(k), V.make_grid(*grid, pairs))
    vd = to_dev(v)
    kb = math.sqrt(D) * (1 + 2.0 ** -7)
    o0, l0 = V.vdit_attn_fwd(qr, kr, vd)
    o1, l1 = V.vdit_attn_fwd(qr, kr, vd, key_norm_max=kb)
    kc, vc = [kr[:, :4000], kr[:, 4000:]], [vd[:, :4000], vd[:, 4000:]]
    r0, rl0 = V.vdit_attn_fwd(qr, mode="ring", k_chunks=kc, v_chunks=vc)
    r1, rl1 = V.vdit_attn_fwd(qr, mode="ring", k_chunks=kc, v_chunks=vc, key_norm_max=kb)
    # rolling: 3 slots of 3000 tokens, frame 4 (two earlier frames in the window)
    kcache = kr[:, :9000].reshape(1, 3, 3000, H, D).contiguous()
    vcache = vd[:, :9000].reshape(1, 3, 3000, H, D).contiguous()
    qf = qr[:, :3000].contiguous()
    f0, fl0 = V.vdit_attn_fwd(qf, mode="rolling", k_cache=kcache, v_cache=vcache, frame=4)
    f1, fl1 = V.vdit_attn_fwd(qf, mode="rolling", k_cache=kcache, v_cache=vcache, frame=4, key_norm_max=kb)
    o2, l2 = V.vdit_attn_fwd(qr, kr, vd, key_norm_max=1.0e4)
    torch.cuda.synchronize()
    for x, y in ((o0, o1), (l0, l1), (r0, r1), (rl0, rl1), (f0, f1), (fl0, fl1)):
        assert torch.equal(x, y)
    wq, wk = O.rope_qk(q.values, k.values, grid, pairs)
    rows = np.unique(np.concatenate([WL.sample_rows(L, 96, seed=92), [0, L - 1]]))
    wo, wl = O.attention(wq[:, rows], wk, v.values)
    check(from_dev(o2)[:, rows], wo, "bf16", "O (bound 1e4: online maximum, sampled rows)")
    check_lse(from_dev(l2)[:, :, rows], wl, "bf16", "LSE (bound 1e4, sampled rows)")
    check(from_dev(o1)[:, rows], wo, "bf16", "O (caller bound, sampled rows)")


def _sampled_attention(qr64, kr64, v64, rows, scale=None):
    o, l = O.attention(qr64[:, rows], kr64, v64, scale)
    return o, l


@pytest.mark.slow
def test_wan13b_full_layer_sampled_rows():
    w = WL.WORKLOADS[2]
    log("Wan-1.3B layer 32760 x 12 x 128: rope + FULL attention, sampled rows")
    q, k, v = WL.workload_inputs(w)
    qr, kr = V.vdit_rope_qk(to_dev(q), to_dev(k), V.make_grid(*w.grid, w.pairs))
    o, lse = V.vdit_attn_fwd(qr, kr, to_dev(v))
    torch.cuda.synchronize()
    rows = WL.sample_rows(w.tokens, 192, seed=7)
    rows = np.unique(np.concatenate([rows, [0, 255, 256, w.tokens - 1]]))  # tile edges and the tail
    wq, wk = O.rope_qk(q.values, k.values, w.grid, w.pairs)
    wo, wl = _sampled_attention(wq, wk, v.values, rows)
    check(from_dev(o)[:, rows], wo, "bf16", "O (sampled rows)")
    check_lse(from_dev(lse)[:, :, rows], wl, "bf16", "LSE (sampled rows)")


@pytest.mark.slow
def test_wan13b_structured_inputs_sampled_rows():
    w = WL.WORKLOADS[2]
    log("Wan-1.3B layer with spatiotemporally smoothed inputs, sampled rows")
    q, k, v = WL.workload_inputs(w, structured=True)
    qr, kr = V.vdit_rope_qk(to_dev(q), to_dev(k), V.make_grid(*w.grid, w.pairs))
    o, lse = V.vdit_attn_fwd(qr, kr, to_dev(v))
    torch.cuda.synchronize()
    rows = WL.sample_rows(w.tokens, 128, seed=8)
    wq, wk = O.rope_qk(q.values, k.values, w.grid, w.pairs)
    wo, wl = _sampled_attention(wq, wk, v.values, rows)
    check(from_dev(o)[:, rows], wo, "bf16", "O (structured, sampled)")
    check_lse(from_dev(lse)[:, :, rows], wl, "bf16", "LSE (structured, sampled)")


def test_offsets_beyond_2_31_elements():
    """64-bit offsets: q and o hold more than 2^31 bf16 elements (4.4 GB
    each): 65 x 256 x 256 = 4,259,840 tokens, 8 heads, D = 64, attending to
    192 keys.  q is a seeded 4096-token block repeated along the sequence
    (token i holds block row i mod 4096), rotated in place at its own grid
    position; rows at the start, past 2^31 bytes and at the very end are
    checked against the oracle."""
    T, Hg, Wg = 65, 256, 256
    L, H, D, Lk, blk = T * Hg * Wg, 8, 64, 192, 4096
    pairs = (12, 10, 10)
    assert L * H * D > 2 ** 31
    log(f"64-bit offsets: {L} tokens x {H} heads x {D} (q {L * H * D * 2 / 1e9:.2f} GB)")
    qb = raw((1, blk, H, D), 71, "bf16"); k = raw((1, Lk, H, D), 72, "bf16"); v = raw((1, Lk, H, D), 73, "bf16")
    qd = to_dev(qb).repeat(1, L // blk + 1, 1, 1)[:, :L].contiguous()
    kd, vd = to_dev(k), to_dev(v)
    V.vdit_rope_qk(qd, None, V.make_grid(T, Hg, Wg, pairs), q_out=qd)
    kgrid = (3, 8, 8)
    V.vdit_rope_qk(None, kd, V.make_grid(*kgrid, pairs), k_out=kd)
    o, lse = V.vdit_attn_fwd(qd, kd, vd)
    torch.cuda.synchronize()
    rows = np.array([0, 1, 4095, 4096, 2 ** 21 - 1, 2 ** 21, 2 ** 21 + 77, 2 ** 22 - 1, 2 ** 22, L - 4097, L - 2, L - 1])
    rows_d = torch.from_numpy(rows).to("cuda")
    _, wk = O.rope_qk(k.values, k.values, kgrid, pairs)
    wq = np.concatenate([O.rope_qk(qb.values[:, r % blk:r % blk + 1], qb.values[:, :1], (T, Hg, Wg), pairs,
                                   token0=int(r))[0] for r in rows], axis=1)
    check(from_dev(qd.index_select(1, rows_d)), wq, "bf16", "rotated q (sampled rows)")
    wo, wl = O.attention(wq, wk, v.values)
    check(from_dev(o.index_select(1, rows_d)), wo, "bf16", "O (sampled rows)")
    check_lse(from_dev(lse.index_select(2, rows_d)), wl, "bf16", "LSE (sampled rows)")


def test_keys_beyond_2_31_elements():
    """64-bit key offsets: k and v hold more than 2^31 bf16 elements (4.4 GB
    each): a seeded 4096-key block repeated to 4,260,840 keys (8 heads,
    D = 64), attended by 64 queries (the call takes the key split).  The
    first L mod 4096 block keys occur 1041 times, the rest 1040 times, so the
    exact result is the LSE merge of the two key sets' attention with
    ln(multiplicity) added to each LSE (the oracle's own attention and
    merge)."""
    L, H, D, blk, Lq = 65 * 256 * 256 + 1000, 8, 64, 4096, 64
    reps, rem = divmod(L, blk)
    assert rem > 0
    assert L * H * D > 2 ** 31
    log(f"64-bit key offsets: {Lq} queries x {L} keys x {H} heads x {D}")
    q = raw((1, Lq, H, D), 74, "bf16"); kb = raw((1, blk, H, D), 75, "bf16"); vb = raw((1, blk, H, D), 76, "bf16")
    kd = to_dev(kb).repeat(1, reps + 1, 1, 1)[:, :L].contiguous()
    vd = to_dev(vb).repeat(1, reps + 1, 1, 1)[:, :L].contiguous()
    o, lse = V.vdit_attn_fwd(to_dev(q), kd, vd)
    torch.cuda.synchronize()
    oa, la = O.attention(q.values, kb.values[:, :rem], vb.values[:, :rem])
    ob, lb = O.attention(q.values, kb.values[:, rem:], vb.values[:, rem:])
    wo, wl = O.lse_merge(oa, la + np.log(reps + 1), ob, lb + np.log(reps))
    check(o, wo, "bf16", "O")
    check_lse(lse, wl, "bf16", "LSE")


def test_attention_deterministic():
    log("determinism: two FULL runs bitwise equal")
    q = raw((1, 600, 4, 128), 51, "bf16"); k = raw((1, 700, 4, 128), 52, "bf16"); v = raw((1, 700, 4, 128), 53, "bf16")
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    o1, l1 = V.vdit_attn_fwd(qd, kd, vd)
    o2, l2 = V.vdit_attn_fwd(qd, kd, vd)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_concurrent_streams_equal_serial():
    """No shared mutable state between calls: FULL (with its key split and
    key-norm pass) and RING calls issued on two streams at once give the
    same bits as the same calls one after the other."""
    log("two streams: FULL and RING concurrently == serially")
    q = raw((1, 900, 4, 128), 61, "bf16"); k = raw((1, 2100, 4, 128), 62, "bf16"); v = raw((1, 2100, 4, 128), 63, "bf16")
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    kc = [kd[:, :1000], kd[:, 1000:]]; vc = [vd[:, :1000], vd[:, 1000:]]
    o_full, l_full = V.vdit_attn_fwd(qd, kd, vd)
    o_ring, l_ring = V.vdit_attn_fwd(qd, mode="ring", k_chunks=kc, v_chunks=vc)
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    s1.wait_stream(torch.cuda.current_stream()); s2.wait_stream(torch.cuda.current_stream())
    outs = []
    for _ in range(3):
        with torch.cuda.stream(s1):
            a = V.vdit_attn_fwd(qd, kd, vd)
        with torch.cuda.stream(s2):
            b = V.vdit_attn_fwd(qd, mode="ring", k_chunks=kc, v_chunks=vc)
        outs.append((a, b))
    torch.cuda.synchronize()
    for (oa, la), (ob, lb) in outs:
        assert torch.equal(oa, o_full) and torch.equal(la, l_full)
        assert torch.equal(ob, o_ring) and torch.equal(lb, l_ring)


# --------------------------------------------------------------------- ring --

@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_ring_small_with_empty_chunk(dtype):
    log(f"ring: 4 chunks incl. an empty one, {dtype}")
    D = 128 if dtype == "bf16" else 64
    q = raw((1, 280, 2, D), 61, dtype)
    lens = [100, 0, 157, 65]
    ks = [raw((1, n, 2, D), 62 + i, dtype) for i, n in enumerate(lens)]
    vs = [raw((1, n, 2, D), 72 + i, dtype) for i, n in enumerate(lens)]
    o, lse = V.vdit_attn_fwd(to_dev(q), mode="ring", k_chunks=[to_dev(x) for x in ks],
                             v_chunks=[to_dev(x) for x in vs])
    torch.cuda.synchronize()
    K = np.concatenate([x.values for x in ks], axis=1); Vv = np.concatenate([x.values for x in vs], axis=1)
    wo, wl = O.attention(q.values, K, Vv)
    check(o, wo, dtype, "O ring"); check_lse(lse, wl, dtype, "LSE ring")
    # reduction-order equivalence: ring == full on the concatenation
    of, lf = V.vdit_attn_fwd(to_dev(q), torch.from_numpy(K.astype(np.float32)).to(o.dtype).cuda(),
                             torch.from_numpy(Vv.astype(np.float32)).to(o.dtype).cuda())
    torch.cuda.synchronize()
    check(o, from_dev(of), dtype, "ring vs full (GPU)")


def test_ring_one_launch_and_fold_forms():
    # bf16 rings of 2..8 chunks run in one launch (a float32 partial per chunk,
    # then the split merge) when the workspace holds the partials, else one
    # launch per chunk folded into the running partial; more chunks always fold
    D, Hq, Hk = 128, 4, 2
    log("ring: one-launch form vs fold form (4 chunks, one empty) and a 9-chunk ring")
    q = raw((1, 300, Hq, D), 171, "bf16")
    lens = [100, 0, 157, 65]
    ks = [raw((1, n, Hk, D), 172 + i, "bf16") for i, n in enumerate(lens)]
    vs = [raw((1, n, Hk, D), 182 + i, "bf16") for i, n in enumerate(lens)]
    kd, vd = [to_dev(x) for x in ks], [to_dev(x) for x in vs]
    align = lambda x: (x + 255) // 256 * 256
    required = align(300 * Hq * D * 4) + align(Hq * 300 * 4)
    o1, l1 = V.vdit_attn_fwd(to_dev(q), mode="ring", k_chunks=kd, v_chunks=vd)
    o2, l2 = V.vdit_attn_fwd(to_dev(q), mode="ring", k_chunks=kd, v_chunks=vd,
                             workspace=torch.empty(required, dtype=torch.uint8, device="cuda"))
    torch.cuda.synchronize()
    wo, wl = O.attention(q.values, np.concatenate([x.values for x in ks], 1), np.concatenate([x.values for x in vs], 1))
    check(o1, wo, "bf16", "O ring, one launch"); check_lse(l1, wl, "bf16", "LSE ring, one launch")
    check(o2, wo, "bf16", "O ring, folded"); check_lse(l2, wl, "bf16", "LSE ring, folded")
    lens9 = [37, 64, 0, 129, 5, 77, 64, 1, 90]
    ks = [raw((1, n, Hk, D), 190 + i, "bf16") for i, n in enumerate(lens9)]
    vs = [raw((1, n, Hk, D), 200 + i, "bf16") for i, n in enumerate(lens9)]
    o9, l9 = V.vdit_attn_fwd(to_dev(q), mode="ring", k_chunks=[to_dev(x) for x in ks], v_chunks=[to_dev(x) for x in vs])
    torch.cuda.synchronize()
    wo, wl = O.attention(q.values, np.concatenate([x.values for x in ks], 1), np.concatenate([x.values for x in vs], 1))
    check(o9, wo, "bf16", "O ring, 9 chunks"); check_lse(l9, wl, "bf16", "LSE ring, 9 chunks")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_batch_of_two_ring_rolling_hybrid(dtype):
    # B = 2 in the modes whose tensors carry more than [B, L, H, D]: ring
    # chunks, the batch-major rolling cache [B, n_slots, L, Hk, D], and the
    # per-(batch, kv head) hybrid state; grouped-query heads throughout
    D, Hq, Hk = (128, 4, 2) if dtype == "bf16" else (64, 4, 1)
    log(f"batch of two: ring, rolling, hybrid {dtype} D={D} Hq={Hq} Hk={Hk}")
    # ring
    q = raw((2, 150, Hq, D), 141, dtype)
    lens = [70, 91]
    ks = [raw((2, n, Hk, D), 142 + i, dtype) for i, n in enumerate(lens)]
    vs = [raw((2, n, Hk, D), 144 + i, dtype) for i, n in enumerate(lens)]
    o, lse = V.vdit_attn_fwd(to_dev(q), mode="ring", k_chunks=[to_dev(x) for x in ks],
                             v_chunks=[to_dev(x) for x in vs])
    torch.cuda.synchronize()
    wo, wl = O.attention(q.values, np.concatenate([x.values for x in ks], 1), np.concatenate([x.values for x in vs], 1))
    check(o, wo, dtype, "O ring B=2"); check_lse(lse, wl, dtype, "LSE ring B=2")
    # rolling: 4 frames through a 2-slot cache, frames handed in by the call
    F, L, W = 4, 77, 2
    qf = raw((F, 2, L, Hq, D), 151, dtype); kf = raw((F, 2, L, Hk, D), 152, dtype); vf = raw((F, 2, L, Hk, D), 153, dtype)
    qd, kd, vd = to_dev(qf), to_dev(kf), to_dev(vf)
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    kc = torch.zeros((2, W, L, Hk, D), dtype=dt, device="cuda"); vc = torch.zeros_like(kc)
    for f in range(F):
        o, lse = V.vdit_attn_fwd(qd[f].contiguous(), kd[f].contiguous(), vd[f].contiguous(), mode="rolling",
                                 k_cache=kc, v_cache=vc, frame=f)
        torch.cuda.synchronize()
        win = list(O.rolling_window(f, W))
        K = np.concatenate([kf.values[u] for u in win], 1); Vv = np.concatenate([vf.values[u] for u in win], 1)
        wo, wl = O.attention(qf.values[f], K, Vv)
        check(o, wo, dtype, f"O rolling B=2 frame {f}"); check_lse(lse, wl, dtype, f"LSE rolling B=2 frame {f}")
    # hybrid with overlap and an incoming state
    L, C, Ov = 180, 48, 24
    q = raw((2, L, Hq, D), 161, dtype); k = raw((2, L, Hk, D), 162, dtype); v = raw((2, L, Hk, D), 163, dtype)
    rng = np.random.default_rng(164)
    s0 = (0.05 * rng.standard_normal((2, Hk, D, D))).astype(np.float32)
    z0 = np.abs(rng.standard_normal((2, Hk, D))).astype(np.float32)
    sd = torch.from_numpy(s0).cuda(); zd = torch.from_numpy(z0).cuda()
    o, lse = V.vdit_attn_fwd(to_dev(q), to_dev(k), to_dev(v), mode="hybrid", chunk_tokens=C, state_s=sd,
                             state_z=zd, overlap_tokens=Ov)
    torch.cuda.synchronize()
    wo, wl, ws_, wz = O.hybrid_recurrent(q.values, k.values, v.values, C, s0=s0, z0=z0, overlap=Ov)
    check(o, wo, dtype, "O hybrid B=2"); check_lse(lse, wl, dtype, "LSE hybrid B=2")
    rs = np.linalg.norm(from_dev(sd) - ws_) / np.linalg.norm(ws_)
    rz = np.linalg.norm(from_dev(zd) - wz) / np.linalg.norm(wz)
    assert rs <= 1e-5 and rz <= 1e-5, (rs, rz)


@pytest.mark.slow
@pytest.mark.parametrize("half,fold", [(0, True), (0, False), (1, True)])
def test_ring_shard_14b_sampled_rows(half, fold):
    # the query shard is frames 0-9 (the first half) or frames 10-19 (the
    # second) of the 20 x 30 x 52 grid; the ring folds the two key chunks in
    # order (the ring step's form) or attends to both in one launch
    w = WL.WORKLOADS[3]
    log(f"14B-shaped shard: Q = half {half} (15600), K/V 2 x 15600, 10 heads, ring of 2 + LSE merge, "
        f"{'fold' if fold else 'one launch'}, sampled rows")
    q, k, v = WL.workload_inputs(w)
    g = V.make_grid(*w.grid, w.pairs)
    q0, q1 = half * w.q_range[1], w.q_range[1]
    qd = to_dev(q)[:, q0:q0 + q1].contiguous()
    kd, vd = to_dev(k), to_dev(v)
    qr, _ = V.vdit_rope_qk(qd, None, g, token0=q0)
    kchunks = []
    for (s, n) in w.kv_chunks:
        _, kc = V.vdit_rope_qk(None, kd[:, s:s + n].contiguous(), g, token0=s)
        kchunks.append(kc)
    vchunks = [vd[:, s:s + n].contiguous() for (s, n) in w.kv_chunks]
    o, lse = V.vdit_attn_fwd(qr, mode="ring", k_chunks=kchunks, v_chunks=vchunks, ring_fold=fold)
    torch.cuda.synchronize()
    wq, wk = O.rope_qk(q.values, k.values, w.grid, w.pairs)
    rows = WL.sample_rows(q1, 160, seed=9)
    wo, wl = O.attention(wq[:, q0 + rows], wk, v.values)
    check(from_dev(o)[:, rows], wo, "bf16", "O ring (sampled)")
    check_lse(from_dev(lse)[:, :, rows], wl, "bf16", "LSE ring (sampled)")


# ------------------------------------------------------------------ merge --

@pytest.mark.parametrize("din,dout", [("bf16", "bf16"), ("f32", "bf16"), ("f32", "f32")])
def test_lse_merge(din, dout):
    log(f"lse merge {din}->{dout}")
    B, L, H, D = 2, 37, 3, 128
    oa = raw((B, L, H, D), 81, din); ob = raw((B, L, H, D), 82, din)
    rng = np.random.default_rng(83)
    la = rng.standard_normal((B, H, L)).astype(np.float32) * 3
    lb = rng.standard_normal((B, H, L)).astype(np.float32) * 3
    la[0, 0, :5] = -np.inf
    lb[0, 0, 3:8] = -np.inf
    tdt = torch.bfloat16 if dout == "bf16" else torch.float32
    oo, lo = V.vdit_lse_merge(to_dev(oa), torch.from_numpy(la).cuda(), to_dev(ob), torch.from_numpy(lb).cuda(),
                              out_dtype=tdt)
    torch.cuda.synchronize()
    wo, wl = O.lse_merge(oa.values, la, ob.values, lb)
    check(oo, wo, dout, "O merged", rel=False); check_lse(lo, wl, "f32", "LSE merged")
    # in place into a
    if din == dout:
        ad = to_dev(oa); lad = torch.from_numpy(la).cuda()
        V.vdit_lse_merge(ad, lad, to_dev(ob), torch.from_numpy(lb).cuda(), o_out=ad, lse_out=lad)
        torch.cuda.synchronize()
        check(ad, wo, dout, "O merged in place", rel=False); check_lse(lad, wl, "f32", "LSE in place")


# ---------------------------------------------------------------- rolling --

def _rolling_run(qf, kf, vf, frame_grid, pairs, n_slots, frames, prefill_slot=False, kv_norm=False):
    """Stream steps through rope (absolute t) + ROLLING attention; return outputs per step.

    A step covers frame_grid = (T_step, H, W); step f's sub-frames take the
    absolute temporal positions T_step * f + s.  With kv_norm the keys are
    normalised and rotated, the values normalised and the queries rotated
    only.  prefill_slot: vdit_rope_qkv writes the step's keys and values
    straight into their cache slots; else vdit_rope_qk and vdit_rms_norm give
    them to the attention call, which inserts them."""
    F, L, H, D = qf.values.shape
    Hk = kf.values.shape[2]
    T = frame_grid[0]
    dt = torch.bfloat16 if qf.dtype == "bf16" else torch.float32
    kc = torch.zeros((1, n_slots, L, Hk, D), dtype=dt, device="cuda")
    vc = torch.zeros_like(kc)
    g = V.make_grid(*frame_grid, pairs)
    qdev, kdev, vdev = to_dev(qf), to_dev(kf), to_dev(vf)
    qn = False if kv_norm else None
    outs = {}
    for f in range(frames):
        if prefill_slot:
            # a decode step's inputs in one launch: q rotated, k normalised and
            # rotated into its cache slot, v (normalised under KV-norm) into its
            slot = f % n_slots
            qr, _, _ = V.vdit_rope_qkv(qdev[f:f + 1], kdev[f:f + 1], vdev[f:f + 1], g, k_out=kc[:, slot],
                                       v_out=vc[:, slot], t_offset=T * f, q_norm=qn, v_norm=kv_norm)
            o, lse = V.vdit_attn_fwd(qr, mode="rolling", k_cache=kc, v_cache=vc, frame=f)
        else:
            qr, _ = V.vdit_rope_qk(qdev[f:f + 1], None, g, t_offset=T * f, q_norm=qn)
            _, kr = V.vdit_rope_qk(None, kdev[f:f + 1], g, t_offset=T * f)
            vr = V.vdit_rms_norm(vdev[f:f + 1]) if kv_norm else vdev[f:f + 1].contiguous()
            o, lse = V.vdit_attn_fwd(qr, kr, vr, mode="rolling", k_cache=kc, v_cache=vc, frame=f)
        outs[f] = (o, lse)
    torch.cuda.synchronize()
    return outs


@pytest.mark.parametrize("dtype,prefill", [("bf16", False), ("bf16", True), ("f32", False)])
def test_rolling_small_stream(dtype, prefill):
    frame_grid, pairs, H, D, W, F = (1, 6, 7), (12, 10, 10), 2, 64, 3, 7
    L = 42
    log(f"rolling small stream {dtype} prefill={prefill} W={W} frames={F}")
    rng = np.random.default_rng(91)
    qf = WL.draw((F, L, H, D), rng, dtype); kf = WL.draw((F, L, H, D), rng, dtype); vf = WL.draw((F, L, H, D), rng, dtype)
    outs = _rolling_run(qf, kf, vf, frame_grid, pairs, W, F, prefill)
    for f in range(F):
        wo, wl = O.rolling_frame(qf.values, kf.values, vf.values, f, W, frame_grid, pairs)
        check(outs[f][0], wo, dtype, f"O frame {f}")
        check_lse(outs[f][1], wl, dtype, f"LSE frame {f}")


@pytest.mark.parametrize("dtype,D,frame_grid,prefill", [
    ("bf16", 64, (1, 6, 13), True), ("bf16", 64, (2, 5, 9), False), ("bf16", 128, (2, 5, 9), True),
    ("f32", 64, (2, 5, 9), True)])
def test_rolling_kv_norm_gqa_stream(dtype, D, frame_grid, prefill):
    # FlashDecoder-style decode: 8 query heads per KV head, KV-norm, window of
    # 2 steps; frame_grid[0] = 2 streams steps of two sub-frames each
    pairs = (12, 10, 10) if D == 64 else (22, 21, 21)
    Hq, Hk, W, F = 8, 1, 2, 5
    L = frame_grid[0] * frame_grid[1] * frame_grid[2]
    log(f"rolling KV-norm GQA {dtype} D={D} step grid {frame_grid} prefill={prefill} W={W} steps={F}")
    rng = np.random.default_rng(92)
    qf = WL.draw((F, L, Hq, D), rng, dtype); kf = WL.draw((F, L, Hk, D), rng, dtype)
    vf = WL.draw((F, L, Hk, D), rng, dtype)
    outs = _rolling_run(qf, kf, vf, frame_grid, pairs, W, F, prefill, kv_norm=True)
    for f in range(F):
        wo, wl = O.rolling_frame(qf.values, kf.values, vf.values, f, W, frame_grid, pairs, kv_norm=True)
        check(outs[f][0], wo, dtype, f"O step {f}")
        check_lse(outs[f][1], wl, dtype, f"LSE step {f}")


@pytest.mark.slow
def test_rolling_decode_shape_sampled():
    # the whole 64-frame stream through the 5-slot cache (the ring buffer
    # wraps twelve times), checked on frames across it
    w = WL.WORKLOADS[4]
    F = w.n_frames
    log(f"rolling decode 2040 tokens x 16 heads x 64, 5 slots, {F} frames, sampled rows")
    qf, kf, vf = WL.workload_inputs(w)
    outs = _rolling_run(qf, kf, vf, w.grid, w.pairs, w.n_slots, F)
    rows = WL.sample_rows(w.tokens, 96, seed=10)
    for f in (0, 3, 4, 7, 31, 62, 63):
        wo, wl = _rolling_oracle_rows(qf, kf, vf, f, w, rows)
        check(from_dev(outs[f][0])[:, rows], wo, "bf16", f"O frame {f} (sampled)")
        check_lse(from_dev(outs[f][1])[:, :, rows], wl, "bf16", f"LSE frame {f} (sampled)")


@pytest.mark.slow
@pytest.mark.parametrize("number,steps,check_at", [(6, 4, (0, 1, 3)), (7, 3, (0, 2))])
def test_flashdecoder_xl_rolling_sampled(number, steps, check_at):
    # FlashDecoder-XL at 720p: 3600 tokens per frame, 24 query heads in 3 KV
    # groups, head dim 64, KV-norm, window of 2; workload 7 is its temporal
    # refinement (steps of 4 sub-frames = 14400 tokens, window of 8 sub-frames)
    w = WL.WORKLOADS[number]
    log(f"{w.name}: {w.tokens} tokens per step x {w.heads}/{w.kv_heads} heads x {w.head_dim}, "
        f"{w.n_slots} slots, {steps} steps, sampled rows")
    q, k, v = WL.workload_inputs(w)
    sub = lambda t: WL.Tensor(t.values[:steps], None if t.bits is None else t.bits[:steps], t.dtype)
    qf, kf, vf = sub(q), sub(k), sub(v)
    del q, k, v
    outs = _rolling_run(qf, kf, vf, w.grid, w.pairs, w.n_slots, steps, prefill_slot=True, kv_norm=w.kv_norm)
    rows = WL.sample_rows(w.tokens, 96, seed=11)
    for f in check_at:
        wo, wl = _rolling_oracle_rows(qf, kf, vf, f, w, rows)
        check(from_dev(outs[f][0])[:, rows], wo, "bf16", f"O step {f} (sampled)")
        check_lse(from_dev(outs[f][1])[:, :, rows], wl, "bf16", f"LSE step {f} (sampled)")


def _rolling_oracle_rows(qf, kf, vf, f, w, rows):
    """oracle.rolling_frame restricted to a sample of query rows (window-relative t,
    T_step temporal positions per step; KV-norm when the workload has it)."""
    win = list(O.rolling_window(f, w.n_slots))
    f0, T = win[0], w.grid[0]
    ks, vs = [], []
    for u in win:
        _, ku = O.rope_qk(kf.values[u][None], kf.values[u][None], w.grid, w.pairs, t_offset=T * (u - f0))
        ks.append(ku)
        vs.append(O.rmsnorm(vf.values[u][None]) if w.kv_norm else vf.values[u][None])
    qr, _ = O.rope_qk(qf.values[f][None], qf.values[f][None], w.grid, w.pairs, t_offset=T * (f - f0),
                      q_norm=False if w.kv_norm else None)
    return O.attention(qr[:, rows], np.concatenate(ks, 1), np.concatenate(vs, 1))


# ----------------------------------------------------------------- hybrid --

@pytest.mark.parametrize("dtype,D,L,C,Hq,Hk", [
    ("bf16", 128, 300, 72, 2, 2), ("bf16", 64, 260, 64, 4, 2), ("bf16", 128, 50, 100, 2, 1),
    ("f32", 64, 100, 24, 2, 1), ("f32", 128, 70, 16, 2, 2),
])
def test_hybrid_small(dtype, D, L, C, Hq, Hk):
    log(f"chunk hybrid {dtype} D={D} L={L} chunk={C} Hq={Hq} Hk={Hk}")
    q = raw((1, L, Hq, D), 101, dtype); k = raw((1, L, Hk, D), 102, dtype); v = raw((1, L, Hk, D), 103, dtype)
    rng = np.random.default_rng(104)
    s0 = (0.05 * rng.standard_normal((1, Hk, D, D))).astype(np.float32)
    z0 = np.abs(rng.standard_normal((1, Hk, D))).astype(np.float32)
    sd = torch.from_numpy(s0).cuda(); zd = torch.from_numpy(z0).cuda()
    o, lse = V.vdit_attn_fwd(to_dev(q), to_dev(k), to_dev(v), mode="hybrid", chunk_tokens=C,
                             state_s=sd, state_z=zd)
    torch.cuda.synchronize()
    wo, wl, ws_, wz = O.hybrid_recurrent(q.values, k.values, v.values, C, s0=s0, z0=z0)
    check(o, wo, dtype, "O hybrid"); check_lse(lse, wl, dtype, "LSE hybrid")
    # state: float32 accumulation of many terms -> relative check
    gs, gz = from_dev(sd), from_dev(zd)
    rs = np.linalg.norm(gs - ws_) / np.linalg.norm(ws_)
    rz = np.linalg.norm(gz - wz) / np.linalg.norm(wz)
    log(f"  state relF s={rs:.3e} z={rz:.3e}")
    assert rs <= 1e-5 and rz <= 1e-5


def test_hybrid_chunkwise_calls_equal_one_call():
    log("chunk hybrid: one call per chunk == one call")
    D, L, C, H = 128, 256, 64, 2
    q = raw((1, L, H, D), 111, "bf16"); k = raw((1, L, H, D), 112, "bf16"); v = raw((1, L, H, D), 113, "bf16")
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    s1 = torch.zeros((1, H, D, D), device="cuda"); z1 = torch.zeros((1, H, D), device="cuda")
    o1, _ = V.vdit_attn_fwd(qd, kd, vd, mode="hybrid", chunk_tokens=C, state_s=s1, state_z=z1)
    s2 = torch.zeros_like(s1); z2 = torch.zeros_like(z1)
    parts = []
    for c0 in range(0, L, C):
        sl = slice(c0, c0 + C)
        oc, _ = V.vdit_attn_fwd(qd[:, sl].contiguous(), kd[:, sl].contiguous(), vd[:, sl].contiguous(),
                                mode="hybrid", chunk_tokens=C, state_s=s2, state_z=z2)
        parts.append(oc)
    torch.cuda.synchronize()
    o2 = torch.cat(parts, dim=1)
    assert torch.equal(o1, o2), float((o1.float() - o2.float()).abs().max())
    assert torch.equal(s1, s2) and torch.equal(z1, z2)


@pytest.mark.parametrize("dtype,D,L,C,Ov,Hq,Hk", [
    ("bf16", 128, 300, 72, 36, 2, 2), ("bf16", 64, 260, 64, 100, 4, 2), ("bf16", 128, 200, 64, 200, 2, 1),
    ("f32", 64, 100, 24, 12, 2, 1), ("f32", 128, 70, 16, 40, 2, 2),
])
def test_hybrid_overlap_small(dtype, D, L, C, Ov, Hq, Hk):
    # softmax windows reaching Ov keys before each chunk (wider than a chunk,
    # or covering everything); the linear state covers the keys before them
    log(f"chunk hybrid with overlap {dtype} D={D} L={L} chunk={C} overlap={Ov} Hq={Hq} Hk={Hk}")
    q = raw((1, L, Hq, D), 121, dtype); k = raw((1, L, Hk, D), 122, dtype); v = raw((1, L, Hk, D), 123, dtype)
    rng = np.random.default_rng(124)
    s0 = (0.05 * rng.standard_normal((1, Hk, D, D))).astype(np.float32)
    z0 = np.abs(rng.standard_normal((1, Hk, D))).astype(np.float32)
    sd = torch.from_numpy(s0).cuda(); zd = torch.from_numpy(z0).cuda()
    o, lse = V.vdit_attn_fwd(to_dev(q), to_dev(k), to_dev(v), mode="hybrid", chunk_tokens=C,
                             state_s=sd, state_z=zd, overlap_tokens=Ov)
    torch.cuda.synchronize()
    wo, wl, ws_, wz = O.hybrid_recurrent(q.values, k.values, v.values, C, s0=s0, z0=z0, overlap=Ov)
    check(o, wo, dtype, "O hybrid"); check_lse(lse, wl, dtype, "LSE hybrid")
    gs, gz = from_dev(sd), from_dev(zd)
    rs = np.linalg.norm(gs - ws_) / np.linalg.norm(ws_)
    rz = np.linalg.norm(gz - wz) / np.linalg.norm(wz)
    log(f"  state relF s={rs:.3e} z={rz:.3e}")
    assert rs <= 1e-5 and rz <= 1e-5


def test_hybrid_overlap_streaming_calls_equal_one_call():
    # calls on chunk boundaries, each after the first carrying the previous
    # overlap keys/values as context, equal one call (bit for bit) and the oracle
    log("chunk hybrid with overlap: streaming calls with context == one call")
    D, L, C, Ov, H = 128, 320, 64, 32, 2
    q = raw((1, L, H, D), 131, "bf16"); k = raw((1, L, H, D), 132, "bf16"); v = raw((1, L, H, D), 133, "bf16")
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    s1 = torch.zeros((1, H, D, D), device="cuda"); z1 = torch.zeros((1, H, D), device="cuda")
    o1, l1 = V.vdit_attn_fwd(qd, kd, vd, mode="hybrid", chunk_tokens=C, state_s=s1, state_z=z1,
                             overlap_tokens=Ov)
    s2 = torch.zeros_like(s1); z2 = torch.zeros_like(z1)
    parts = []
    for a, b in ((0, 128), (128, 192), (192, 320)):
        c = min(Ov, a)
        oc, _ = V.vdit_attn_fwd(qd[:, a:b].contiguous(), kd[:, a - c:b].contiguous(), vd[:, a - c:b].contiguous(),
                                mode="hybrid", chunk_tokens=C, state_s=s2, state_z=z2, overlap_tokens=Ov,
                                ctx_tokens=c)
        parts.append(oc)
    torch.cuda.synchronize()
    o2 = torch.cat(parts, dim=1)
    assert torch.equal(o1, o2), float((o1.float() - o2.float()).abs().max())
    assert torch.equal(s1, s2) and torch.equal(z1, z2)
    wo, wl, ws_, _ = O.hybrid_recurrent(q.values, k.values, v.values, C, overlap=Ov)
    check(o1, wo, "bf16", "O hybrid"); check_lse(l1, wl, "bf16", "LSE hybrid")
    rs = np.linalg.norm(from_dev(s1) - ws_) / np.linalg.norm(ws_)
    assert rs <= 1e-5, rs


@pytest.mark.slow
def test_hybrid_overlap_full_c4_o2():
    # chunks of T_c = 4 latent frames (1560 tokens) with T_o = 2 frames (780
    # tokens) of softmax overlap on the 31 x 15 x 26 grid, all rows
    w = WL.WORKLOADS[8]
    log(f"{w.name}: rope + hybrid (chunk {w.chunk_tokens}, overlap {w.overlap_tokens}) vs oracle (all rows)")
    q, k, v = WL.workload_inputs(w)
    qr, kr = V.vdit_rope_qk(to_dev(q), to_dev(k), V.make_grid(*w.grid, w.pairs))
    sd = torch.zeros((1, w.kv_heads, w.head_dim, w.head_dim), device="cuda")
    zd = torch.zeros((1, w.kv_heads, w.head_dim), device="cuda")
    o, lse = V.vdit_attn_fwd(qr, kr, to_dev(v), mode="hybrid", chunk_tokens=w.chunk_tokens, state_s=sd,
                             state_z=zd, overlap_tokens=w.overlap_tokens)
    torch.cuda.synchronize()
    wq, wk = O.rope_qk(q.values, k.values, w.grid, w.pairs)
    o_s, l_s, o_l, l_l = O.hybrid_partials(wq, wk, v.values, w.chunk_tokens, overlap=w.overlap_tokens)
    wo, wl = O.lse_merge(o_s, l_s, o_l, l_l)
    check(o, wo, "bf16", "O hybrid (all rows)")
    check_lse(lse, wl, "bf16", "LSE hybrid")
    # (the state is checked to 1e-5 on the library's own rotated keys in
    # test_gpu_hybrid.py; here the oracle rotates in float64, end to end)


@pytest.mark.slow
def test_hybrid_5b_full():
    w = WL.WORKLOADS[5]
    log("chunk hybrid 12090 x 24 x 128, chunks of 1170: rope + hybrid vs oracle (all rows)")
    q, k, v = WL.workload_inputs(w)
    qr, kr = V.vdit_rope_qk(to_dev(q), to_dev(k), V.make_grid(*w.grid, w.pairs))
    sd = torch.zeros((1, w.kv_heads, w.head_dim, w.head_dim), device="cuda")
    zd = torch.zeros((1, w.kv_heads, w.head_dim), device="cuda")
    o, lse = V.vdit_attn_fwd(qr, kr, to_dev(v), mode="hybrid", chunk_tokens=w.chunk_tokens, state_s=sd, state_z=zd)
    torch.cuda.synchronize()
    wq, wk = O.rope_qk(q.values, k.values, w.grid, w.pairs)
    o_s, l_s, o_l, l_l = O.hybrid_partials(wq, wk, v.values, w.chunk_tokens)
    wo, wl = O.lse_merge(o_s, l_s, o_l, l_l)
    check(o, wo, "bf16", "O hybrid (all rows)")
    check_lse(lse, wl, "bf16", "LSE hybrid")
    # (the state is checked to 1e-5 on the library's own rotated keys in
    # test_gpu_hybrid.py; here the oracle rotates in float64, end to end)


# ----------------------------------------------------------- graphs ------

def test_graph_capture_replays_equal_eager():
    # The library neither allocates, synchronises nor issues memsets, so its
    # calls can be captured: FULL with the key split (several kernels), the
    # one-launch RING and the hybrid with overlap (state reset by a fill
    # kernel inside the graph).  Every replay, with eager work between them,
    # must equal the eager results bit for bit (no atomics anywhere).
    log("graph capture: FULL (split), RING (one launch), hybrid (overlap), 3 replays")
    qf = to_dev(raw((1, 1000, 2, 128), 221, "bf16"))
    kf = to_dev(raw((1, 5000, 1, 128), 222, "bf16")); vf = to_dev(raw((1, 5000, 1, 128), 223, "bf16"))
    kc = [to_dev(raw((1, n, 2, 64), 224 + i, "bf16")) for i, n in enumerate((300, 450))]
    vc = [to_dev(raw((1, n, 2, 64), 226 + i, "bf16")) for i, n in enumerate((300, 450))]
    qr = to_dev(raw((1, 700, 4, 64), 228, "bf16"))
    qh = to_dev(raw((1, 260, 2, 128), 229, "bf16"))
    kh = to_dev(raw((1, 260, 2, 128), 230, "bf16")); vh = to_dev(raw((1, 260, 2, 128), 231, "bf16"))
    sd = torch.zeros((1, 2, 128, 128), device="cuda"); zd = torch.zeros((1, 2, 128), device="cuda")

    def run():
        o1, l1 = V.vdit_attn_fwd(qf, kf, vf)
        o2, l2 = V.vdit_attn_fwd(qr, mode="ring", k_chunks=kc, v_chunks=vc)
        sd.zero_(); zd.zero_()
        o3, l3 = V.vdit_attn_fwd(qh, kh, vh, mode="hybrid", chunk_tokens=64, state_s=sd, state_z=zd,
                                 overlap_tokens=32)
        return [o1, l1, o2, l2, o3, l3, sd, zd]

    eager = [t.clone() for t in run()]
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        outs = run()
    for rep in range(3):
        V.vdit_attn_fwd(qf, kf, vf)  # eager work between replays
        torch.cuda.synchronize()
        for t in outs:
            t.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        for j, (a, b) in enumerate(zip(outs, eager)):
            assert torch.equal(a, b), (rep, j, float((a.float() - b.float()).abs().max()))


# -------------------------------------------------------- C consumer ------

def test_c_abi_consumer_program(tmp_path):
    # tests/host/c_consumer.c uses the library as a C program would (hipMalloc,
    # its own stream, workspace from vdit_attn_workspace_bytes, statuses):
    # RMSNorm + 3D-RoPE (also with the values normalised in the same launch,
    # whose q and k it compares with the first call's bit for bit), FULL and
    # a two-chunk RING, checked against the oracle
    from video_diffusion_transformer_rmsnorm_amd import build as B
    if not os.path.exists(B.CONSUMER):
        pytest.fail(f"{B.CONSUMER} is not built (run __graft_entry__.build())")
    grid, pairs, Hq, Hk, D, split = (3, 10, 17), (22, 21, 21), 4, 2, 128, 200
    L = grid[0] * grid[1] * grid[2]
    log(f"C consumer: L={L} Hq={Hq} Hk={Hk} D={D}, ring split at {split}")
    rng = np.random.default_rng(211)
    q = WL.draw((1, L, Hq, D), rng, "bf16"); k = WL.draw((1, L, Hk, D), rng, "bf16"); v = WL.draw((1, L, Hk, D), rng, "bf16")
    for name, t in (("q.bin", q), ("k.bin", k), ("v.bin", v)):
        np.ascontiguousarray(t.bits).tofile(str(tmp_path / name))
    (tmp_path / "meta.txt").write_text(f"{L} {Hq} {Hk} {D} {grid[0]} {grid[1]} {grid[2]} {pairs[0]} {pairs[1]} {pairs[2]} {split}\n")
    r = subprocess.run([B.CONSUMER, str(tmp_path)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and "c_consumer ok" in r.stdout, r.stdout + r.stderr
    bf = lambda name, shape: WL.bf16_bits_to_f64(np.fromfile(str(tmp_path / name), dtype=np.uint16)).reshape(shape)
    f32 = lambda name, shape: np.fromfile(str(tmp_path / name), dtype=np.float32).astype(np.float64).reshape(shape)
    wq, wk = O.rope_qk(q.values, k.values, grid, pairs)
    check(bf("qr.bin", (1, L, Hq, D)), wq, "bf16", "q rotated (C)")
    check(bf("kr.bin", (1, L, Hk, D)), wk, "bf16", "k rotated (C)")
    wo, wl = O.attention(wq, wk, v.values)
    check(bf("o_full.bin", (1, L, Hq, D)), wo, "bf16", "O full (C)")
    check_lse(f32("lse_full.bin", (1, Hq, L)), wl, "bf16", "LSE full (C)")
    check(bf("o_ring.bin", (1, L, Hq, D)), wo, "bf16", "O ring (C)")
    check_lse(f32("lse_ring.bin", (1, Hq, L)), wl, "bf16", "LSE ring (C)")
    check(bf("vn.bin", (1, L, Hk, D)), O.rmsnorm(v.values), "bf16", "v normalised by vdit_rope_qkv (C)")


# ------------------------------------------------------------ randomised --

def _random_case(i):
    """Seeded configuration i: mode, dtype, head dim, GQA ratio and ragged sizes."""
    r = np.random.default_rng(5000 + i)
    mode = ["full", "ring", "rolling", "hybrid"][i % 4]
    dtype = "bf16" if r.random() < 0.75 else "f32"
    D = int(r.choice([64, 128]))
    Hk = int(r.choice([1, 2, 3]))
    Hq = Hk * int(r.choice([1, 2, 4, 8]))
    return r, mode, dtype, D, Hq, Hk


@pytest.mark.parametrize("i", range(24))
def test_randomised_configurations(i):
    r, mode, dtype, D, Hq, Hk = _random_case(i)
    B = int(r.choice([1, 2]))
    seed = 6000 + 10 * i
    if mode == "full":
        Lq, Lkv = int(r.integers(1, 700)), int(r.integers(0, 1500))
        log(f"random {i}: full {dtype} D={D} B={B} Lq={Lq} Lkv={Lkv} Hq={Hq} Hk={Hk}")
        q = raw((B, Lq, Hq, D), seed, dtype); k = raw((B, Lkv, Hk, D), seed + 1, dtype); v = raw((B, Lkv, Hk, D), seed + 2, dtype)
        kd = to_dev(k) if Lkv else torch.empty((B, 0, Hk, D), dtype=torch.bfloat16 if dtype == "bf16" else torch.float32, device="cuda")
        vd = to_dev(v) if Lkv else kd
        o, lse = V.vdit_attn_fwd(to_dev(q), kd, vd)
        torch.cuda.synchronize()
        if Lkv == 0:
            assert (from_dev(o) == 0).all() and np.isneginf(from_dev(lse)).all()
            return
        wo, wl = O.attention(q.values, k.values, v.values)
    elif mode == "ring":
        Lq = int(r.integers(1, 500))
        lens = [int(x) for x in r.integers(0, 300, size=int(r.integers(1, 11)))]
        lens[int(r.integers(0, len(lens)))] = max(1, lens[0])  # at least one non-empty chunk
        log(f"random {i}: ring {dtype} D={D} B={B} Lq={Lq} chunks={lens} Hq={Hq} Hk={Hk}")
        q = raw((B, Lq, Hq, D), seed, dtype)
        ks = [raw((B, n, Hk, D), seed + 1 + c, dtype) for c, n in enumerate(lens)]
        vs = [raw((B, n, Hk, D), seed + 50 + c, dtype) for c, n in enumerate(lens)]
        dt = torch.bfloat16 if dtype == "bf16" else torch.float32
        dev = lambda t, n: to_dev(t) if n else torch.empty((B, 0, Hk, D), dtype=dt, device="cuda")
        o, lse = V.vdit_attn_fwd(to_dev(q), mode="ring", k_chunks=[dev(x, n) for x, n in zip(ks, lens)],
                                 v_chunks=[dev(x, n) for x, n in zip(vs, lens)])
        torch.cuda.synchronize()
        wo, wl = O.attention(q.values, np.concatenate([x.values for x in ks], 1), np.concatenate([x.values for x in vs], 1))
    elif mode == "rolling":
        L, W, F = int(r.integers(8, 300)), int(r.integers(1, 5)), int(r.integers(1, 7))
        log(f"random {i}: rolling {dtype} D={D} B={B} L={L} slots={W} frames={F} Hq={Hq} Hk={Hk}")
        qf = raw((F, B, L, Hq, D), seed, dtype); kf = raw((F, B, L, Hk, D), seed + 1, dtype); vf = raw((F, B, L, Hk, D), seed + 2, dtype)
        qd, kd, vd = to_dev(qf), to_dev(kf), to_dev(vf)
        kc = torch.zeros((B, W, L, Hk, D), dtype=qd.dtype, device="cuda"); vc = torch.zeros_like(kc)
        for f in range(F):
            o, lse = V.vdit_attn_fwd(qd[f].contiguous(), kd[f].contiguous(), vd[f].contiguous(), mode="rolling",
                                     k_cache=kc, v_cache=vc, frame=f)
        torch.cuda.synchronize()
        win = list(O.rolling_window(F - 1, W))
        wo, wl = O.attention(qf.values[F - 1], np.concatenate([kf.values[u] for u in win], 1),
                             np.concatenate([vf.values[u] for u in win], 1))
    else:
        L, C = int(r.integers(1, 400)), int(r.integers(1, 150))
        Ov = int(r.choice([0, int(r.integers(1, 2 * C))]))
        ctx = int(r.integers(0, Ov + 1))
        log(f"random {i}: hybrid {dtype} D={D} B={B} L={L} chunk={C} overlap={Ov} ctx={ctx} Hq={Hq} Hk={Hk}")
        q = raw((B, L, Hq, D), seed, dtype); k = raw((B, ctx + L, Hk, D), seed + 1, dtype); v = raw((B, ctx + L, Hk, D), seed + 2, dtype)
        s0 = (0.05 * r.standard_normal((B, Hk, D, D))).astype(np.float32)
        z0 = np.abs(r.standard_normal((B, Hk, D))).astype(np.float32)
        sd = torch.from_numpy(s0).cuda(); zd = torch.from_numpy(z0).cuda()
        o, lse = V.vdit_attn_fwd(to_dev(q), to_dev(k), to_dev(v), mode="hybrid", chunk_tokens=C, state_s=sd,
                                 state_z=zd, overlap_tokens=Ov, ctx_tokens=ctx)
        torch.cuda.synchronize()
        wo, wl, ws_, wz = O.hybrid_explicit(q.values, k.values, v.values, C, s0=s0, z0=z0, overlap=Ov, ctx=ctx)
        rs = np.linalg.norm(from_dev(sd) - ws_) / np.linalg.norm(ws_)
        assert rs <= 1e-5, rs
    check(o, wo, dtype, f"O random {i}")
    check_lse(lse, wl, dtype, f"LSE random {i}")


# ----------------------------------------------------------------- errors --

def test_invalid_arguments_raise():
    log("invalid arguments raise VditError")
    q = torch.zeros((1, 10, 3, 128), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((1, 10, 2, 128), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(V.VditError):
        V.vdit_attn_fwd(q, k, k)  # 3 heads over 2 kv heads
    qq = torch.zeros((1, 10, 2, 96), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(V.VditError):
        V.vdit_attn_fwd(qq, qq, qq)
