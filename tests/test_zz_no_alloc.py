"""vdit_attn_fwd_noalloc (the entry point for callers that cannot allocate)
against vdit_attn_fwd with a caller's workspace, through the C ABI: two calls
in a row per mode, the second on a smaller input, every output equal bit for
bit (same kernels, same workspace plan) and within the parity bar of the
oracle.  Also: a call whose required workspace exceeds the scratch is
rejected before anything runs, and a caller's workspace is refused."""
import ctypes

import numpy as np
import pytest
import torch

import oracle as O
import video_diffusion_transformer_rmsnorm_amd as V
import workloads as WL
from parity import check, check_lse, from_dev, log, to_dev

pytestmark = pytest.mark.gpu


def raw(shape, seed):
    return WL.draw(shape, np.random.default_rng(seed), "bf16")


def _same(a, b, what):
    assert torch.equal(a, b), (what, float((a.float() - b.float()).abs().max()))


@pytest.mark.parametrize("L,Lkv", [(3000, 9000), (700, 1500)])
def test_noalloc_full_with_key_split(L, Lkv):
    log(f"noalloc FULL: Lq={L} Lkv={Lkv}")
    H, D = 4, 128
    q, k, v = raw((1, L, H, D), 901), raw((1, Lkv, H, D), 902), raw((1, Lkv, H, D), 903)
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    o1, l1 = V.vdit_attn_fwd(qd, kd, vd)
    o2, l2 = V.vdit_attn_fwd_noalloc(qd, kd, vd)
    torch.cuda.synchronize()
    _same(o1, o2, "O"); _same(l1, l2, "LSE")
    rows = WL.sample_rows(L, 64, seed=L)
    wo, wl = O.attention(q.values[:, rows], k.values, v.values)
    check(from_dev(o2)[:, rows], wo, "bf16", "O noalloc (sampled rows)")
    check_lse(from_dev(l2)[:, :, rows], wl, "bf16", "LSE noalloc")


def test_noalloc_ring_hybrid_rolling_two_calls_shrinking():
    D, H = 128, 4
    for i, (L, C) in enumerate(((2400, 600), (900, 300))):
        log(f"noalloc call {i}: ring / hybrid / rolling, L={L}")
        q, k, v = raw((1, L, H, D), 910 + i), raw((1, L, H, D), 920 + i), raw((1, L, H, D), 930 + i)
        qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
        # RING, fold form (required running partial in the scratch)
        kc, vc = [kd[:, :L // 3], kd[:, L // 3:]], [vd[:, :L // 3], vd[:, L // 3:]]
        r1, rl1 = V.vdit_attn_fwd(qd, mode="ring", k_chunks=kc, v_chunks=vc, ring_fold=True)
        r2, rl2 = V.vdit_attn_fwd_noalloc(qd, mode="ring", k_chunks=kc, v_chunks=vc, ring_fold=True)
        # CHUNK_HYBRID (deltas, per-chunk state, key bounds in the scratch)
        s1 = torch.zeros((1, H, D, D), device="cuda"); z1 = torch.zeros((1, H, D), device="cuda")
        s2 = torch.zeros_like(s1); z2 = torch.zeros_like(z1)
        h1, hl1 = V.vdit_attn_fwd(qd, kd, vd, mode="hybrid", chunk_tokens=C, state_s=s1, state_z=z1)
        h2, hl2 = V.vdit_attn_fwd_noalloc(qd, kd, vd, mode="hybrid", chunk_tokens=C, state_s=s2, state_z=z2)
        # ROLLING frame 2 over 3 slots of L // 3 tokens
        n = L // 3
        cache_k = kd[:, :3 * n].reshape(1, 3, n, H, D).contiguous()
        cache_v = vd[:, :3 * n].reshape(1, 3, n, H, D).contiguous()
        qf = qd[:, :n].contiguous()
        f1, fl1 = V.vdit_attn_fwd(qf, mode="rolling", k_cache=cache_k, v_cache=cache_v, frame=2)
        f2, fl2 = V.vdit_attn_fwd_noalloc(qf, mode="rolling", k_cache=cache_k, v_cache=cache_v, frame=2)
        torch.cuda.synchronize()
        for a, b, what in ((r1, r2, "ring O"), (rl1, rl2, "ring LSE"), (h1, h2, "hybrid O"), (hl1, hl2, "hybrid LSE"),
                           (s1, s2, "hybrid state s"), (z1, z2, "hybrid state z"), (f1, f2, "rolling O"),
                           (fl1, fl2, "rolling LSE")):
            _same(a, b, what)
        wo, wl = O.attention(q.values, k.values, v.values)
        check(r2, wo, "bf16", "ring O noalloc"); check_lse(rl2, wl, "bf16", "ring LSE noalloc")
        wo, wl, ws_, _ = O.hybrid_recurrent(q.values, k.values, v.values, C)
        check(h2, wo, "bf16", "hybrid O noalloc"); check_lse(hl2, wl, "bf16", "hybrid LSE noalloc")
        rs = np.linalg.norm(from_dev(s2) - ws_) / np.linalg.norm(ws_)
        assert rs <= 1e-5, rs
        wo, wl = O.attention(q.values[:, :n], k.values[:, :3 * n], v.values[:, :3 * n])
        check(f2, wo, "bf16", "rolling O noalloc"); check_lse(fl2, wl, "bf16", "rolling LSE noalloc")


def test_noalloc_rejects_oversized_and_caller_workspace():
    log("noalloc: a required workspace beyond the scratch, and a caller's workspace, are refused")
    H, D = 8, 128
    q = torch.zeros((1, 20000, H, D), dtype=torch.bfloat16, device="cuda")  # fold partial: 82 MB > 64 MiB
    k = torch.zeros((1, 100, H, D), dtype=torch.bfloat16, device="cuda")
    o = torch.full_like(q, 7.0)
    with pytest.raises(V.VditError) as e:
        V.vdit_attn_fwd_noalloc(q, mode="ring", k_chunks=[k, k], v_chunks=[k, k], ring_fold=True, o=o)
    assert e.value.status == V.VDIT_ERR_UNSUPPORTED and "scratch" in str(e.value)
    a = V.VditAttnArgs()
    a.mode, a.dtype, a.B, a.n_heads, a.n_kv_heads, a.head_dim = 0, 0, 1, H, H, D
    a.Lq = a.Lkv = 100
    a.q, a.k, a.v, a.o = k.data_ptr(), k.data_ptr(), k.data_ptr(), o.data_ptr()
    ws = torch.empty(1 << 20, dtype=torch.uint8, device="cuda")
    a.workspace, a.workspace_bytes = ws.data_ptr(), ws.numel()
    assert V.lib().vdit_attn_fwd_noalloc(ctypes.byref(a), None) == V.VDIT_ERR_INVALID_ARG
    assert "workspace" in V.lib().vdit_last_error().decode()
    torch.cuda.synchronize()
    assert bool((o == 7.0).all())  # nothing was written


def test_noalloc_step_recorded_in_a_graph():
    """A caller that records its step into a HIP graph (the case the entry
    point is for): RMSNorm + 3D-RoPE into persistent buffers, then the
    no-allocation attention with its keys split in ranges whose partials
    live in the library's scratch.  Replayed three times with eager calls of
    another shape in between (they reuse the same scratch and leave other
    contents in it); every replay equals the eager call bit for bit."""
    log("noalloc: RoPE + key-split attention recorded in a graph, replayed 3 times")
    H, D, L, Lkv = 4, 128, 1500, 1500  # 48 workgroups of 128 queries: the keys are split
    grid, pairs = (1, 1, Lkv), (22, 21, 21)
    q, k, v = raw((1, L, H, D), 951), raw((1, Lkv, H, D), 952), raw((1, Lkv, H, D), 953)
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    g = V.make_grid(*grid, pairs)
    qr, kr = torch.empty_like(qd), torch.empty_like(kd)
    o_e, l_e = torch.empty_like(qd), torch.empty((1, H, L), dtype=torch.float32, device="cuda")
    o_g, l_g = torch.empty_like(qd), torch.empty_like(l_e)

    def step(o, lse):
        V.vdit_rope_qk(qd, kd, g, q_out=qr, k_out=kr)
        V.vdit_attn_fwd_noalloc(qr, kr, vd, o=o, lse=lse)

    step(o_e, l_e)  # eager reference (also the library's first call on this device)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(o_g, l_g)  # warm-up on a side stream before the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(o_g, l_g)
    other_q, other_k = torch.randn((1, 300, H, D), device="cuda").to(torch.bfloat16), torch.randn(
        (1, 2000, H, D), device="cuda").to(torch.bfloat16)
    for rep in range(3):
        o_g.fill_(float("nan")); l_g.fill_(float("nan"))
        V.vdit_attn_fwd_noalloc(other_q, other_k, other_k)  # eager, same scratch
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        _same(o_g, o_e, f"O replay {rep}"); _same(l_g, l_e, f"LSE replay {rep}")
    wq, wk = O.rope_qk(q.values, k.values, grid, pairs)
    wo, wl = O.attention(wq, wk, v.values)
    check(o_g, wo, "bf16", "O of the replayed graph"); check_lse(l_g, wl, "bf16", "LSE of the replayed graph")
