"""The pipelined attention kernel against its self-check build.

libvdit_debugsync.so is the same source built with VDIT_DEBUG_SYNC=1: every
tile load is waited for before the LDS reads of its iteration and each region
of the software pipeline ends on a workgroup barrier, so no LDS write can
overlap a read of the same bytes.  The arithmetic and its order are
unchanged, so a pipelined build free of LDS hazards gives the same bits.
Every workgroup shape (8, 4 and 2 wavefronts), both softmax paths, the key
split, both ring forms, the rolling window and the hybrid epilogue are
compared, at both head dimensions."""
import contextlib

import numpy as np
import pytest
import torch

import video_diffusion_transformer_rmsnorm_amd as V
from video_diffusion_transformer_rmsnorm_amd import build as B
import workloads as WL
from parity import log, to_dev

pytestmark = pytest.mark.gpu


@contextlib.contextmanager
def debug_library():
    handle = V.load(B.DEBUG_SYNC_LIB)
    saved = V._lib_handle
    V._lib_handle = handle
    try:
        yield
    finally:
        V._lib_handle = saved


def raw(shape, seed):
    return WL.draw(shape, np.random.default_rng(seed), "bf16")


def _calls(D):
    pairs = (22, 21, 21) if D == 128 else (12, 10, 10)
    H, Hk = 8, 2
    out = []

    def full(L, Lkv, seed, **kw):
        q, k, v = raw((1, L, H, D), seed), raw((1, Lkv, Hk, D), seed + 1), raw((1, Lkv, Hk, D), seed + 2)
        g = V.make_grid(1, 1, max(L, Lkv), pairs)
        qd, _ = V.vdit_rope_qk(to_dev(q), None, g)
        _, kd = V.vdit_rope_qk(None, to_dev(k), g)
        return qd, kd, to_dev(v)

    # 256-query (8 wavefronts, bounded) and 128-query (4, bounded) FULL, both
    # with the online maximum too (no workspace for the bound)
    for L in (16347, 9001):
        qd, kd, vd = full(L, 3001, 800 + L)
        out.append(("full", dict(q=qd, k=kd, v=vd)))
        out.append(("full online", dict(q=qd, k=kd, v=vd, workspace=torch.empty(16, dtype=torch.uint8, device="cuda"))))
    # 64-query workgroups with the key split, and unsplit
    qd, kd, vd = full(700, 5000, 810)
    out.append(("full split", dict(q=qd, k=kd, v=vd)))
    out.append(("full small", dict(q=qd, k=kd, v=vd, workspace=torch.empty(16, dtype=torch.uint8, device="cuda"))))
    # ring: one launch and fold
    qd, kd, vd = full(4000, 6000, 820)
    kc, vc = [kd[:, :2500], kd[:, 2500:]], [vd[:, :2500], vd[:, 2500:]]
    out.append(("ring one launch", dict(q=qd, mode="ring", k_chunks=kc, v_chunks=vc)))
    out.append(("ring fold", dict(q=qd, mode="ring", k_chunks=kc, v_chunks=vc, ring_fold=True)))
    # rolling frame 3 of a 3-slot cache
    cache_k = kd[:, :6000].reshape(1, 3, 2000, Hk, D).contiguous()
    cache_v = vd[:, :6000].reshape(1, 3, 2000, Hk, D).contiguous()
    out.append(("rolling", dict(q=qd[:, :2000].contiguous(), mode="rolling", k_cache=cache_k, v_cache=cache_v,
                                frame=3)))
    # hybrid with overlap, and without (a bound per chunk)
    qh, kh, vh = full(3000, 3000, 830)
    for ov in (0, 200):
        out.append((f"hybrid overlap {ov}", dict(q=qh, k=kh, v=vh, mode="hybrid", chunk_tokens=700, overlap_tokens=ov,
                                                 state_s="s", state_z="z")))
    return out, Hk


def _run(kw, Hk, D):
    kw = dict(kw)
    extra = []
    if kw.get("state_s") == "s":
        kw["state_s"] = torch.zeros((1, Hk, D, D), device="cuda")
        kw["state_z"] = torch.zeros((1, Hk, D), device="cuda")
        extra = [kw["state_s"], kw["state_z"]]
    q = kw.pop("q")
    o, lse = V.vdit_attn_fwd(q, **kw)
    torch.cuda.synchronize()
    return [o, lse] + extra


@pytest.mark.parametrize("D", [128, 64])
def test_pipelined_equals_self_check_build(D):
    calls, Hk = _calls(D)
    for name, kw in calls:
        log(f"D={D} {name}")
        a = _run(kw, Hk, D)
        with debug_library():
            b = _run(kw, Hk, D)
        for x, y in zip(a, b):
            assert torch.equal(x, y), (name, float((x.float() - y.float()).abs().max()))
