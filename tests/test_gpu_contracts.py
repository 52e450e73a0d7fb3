"""GPU checks of the ABI's contracts beyond parity: a call that fails
validation writes nothing (not even the parts a valid call would write
first), and a caller's key-norm bound below the true key norms costs time,
never correctness."""
import math

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


def test_rejected_rolling_call_leaves_the_cache_alone():
    # A valid ROLLING call first copies the new frame into its cache slot; a
    # call whose workspace overlaps the cache must be rejected before that copy.
    L, H, D, W = 300, 2, 64, 3
    log(f"rejected ROLLING call: L={L} H={H} D={D} slots={W}")
    q, k, v = (to_dev(raw((1, L, H, D), s)) for s in (301, 302, 303))
    kc = to_dev(raw((1, W, L, H, D), 304)); vc = to_dev(raw((1, W, L, H, D), 305))
    k0, v0 = kc.clone(), vc.clone()
    bad_ws = kc.view(torch.uint8).reshape(-1)[: 1 << 16]
    with pytest.raises(V.VditError, match="overlaps"):
        V.vdit_attn_fwd(q, k, v, mode="rolling", k_cache=kc, v_cache=vc, frame=1, workspace=bad_ws)
    misaligned = torch.empty(4096 + 8, dtype=torch.uint8, device="cuda")[8:]
    with pytest.raises(V.VditError, match="aligned"):
        V.vdit_attn_fwd(q, k, v, mode="rolling", k_cache=kc, v_cache=vc, frame=1, workspace=misaligned)
    torch.cuda.synchronize()
    assert torch.equal(kc, k0) and torch.equal(vc, v0)
    # the same call with a proper workspace inserts the frame and matches the oracle
    o, lse = V.vdit_attn_fwd(q, k, v, mode="rolling", k_cache=kc, v_cache=vc, frame=1)
    torch.cuda.synchronize()
    assert torch.equal(kc[0, 1], k[0]) and torch.equal(vc[0, 1], v[0])
    K = np.concatenate([from_dev(k0[:, 0]), from_dev(k)], 1); Vv = np.concatenate([from_dev(v0[:, 0]), from_dev(v)], 1)
    wo, wl = O.attention(from_dev(q), K, Vv)
    check(o, wo, "bf16", "O rolling after the rejected calls"); check_lse(lse, wl, "bf16", "LSE")


def test_rejected_hybrid_call_leaves_the_state_alone():
    # A valid CHUNK_HYBRID call first folds the keys into the state; a call
    # whose workspace overlaps the state (or o) must be rejected before that.
    L, H, D, C = 256, 2, 128, 64
    log(f"rejected CHUNK_HYBRID call: L={L} H={H} D={D} chunk={C}")
    q, k, v = (to_dev(raw((1, L, H, D), s)) for s in (311, 312, 313))
    rng = np.random.default_rng(314)
    s_init = torch.from_numpy((0.05 * rng.standard_normal((1, H, D, D))).astype(np.float32)).cuda()
    z_init = torch.from_numpy(np.abs(rng.standard_normal((1, H, D))).astype(np.float32)).cuda()
    big = torch.empty(64 << 20, dtype=torch.uint8, device="cuda")
    # a workspace large enough, with the state inside it
    s_in_ws = big[1 << 20:(1 << 20) + s_init.numel() * 4].view(torch.float32).view(s_init.shape)
    s_in_ws.copy_(s_init)
    zd = z_init.clone()
    with pytest.raises(V.VditError, match="overlaps"):
        V.vdit_attn_fwd(q, k, v, mode="hybrid", chunk_tokens=C, state_s=s_in_ws, state_z=zd, workspace=big)
    torch.cuda.synchronize()
    assert torch.equal(s_in_ws, s_init) and torch.equal(zd, z_init)
    sd = s_init.clone()
    s0, z0 = sd.clone(), zd.clone()
    o_in_ws = big[:q.numel() * 2].view(torch.bfloat16).view(q.shape)
    with pytest.raises(V.VditError, match="overlaps"):
        V.vdit_attn_fwd(q, k, v, mode="hybrid", chunk_tokens=C, state_s=sd, state_z=zd, o=o_in_ws, workspace=big)
    torch.cuda.synchronize()
    assert torch.equal(sd, s0) and torch.equal(zd, z0)
    o, lse = V.vdit_attn_fwd(q, k, v, mode="hybrid", chunk_tokens=C, state_s=sd, state_z=zd)
    torch.cuda.synchronize()
    wo, wl, ws_, wz = O.hybrid_recurrent(from_dev(q), from_dev(k), from_dev(v), C, s0=from_dev(s0), z0=from_dev(z0))
    check(o, wo, "bf16", "O hybrid after the rejected calls"); check_lse(lse, wl, "bf16", "LSE")
    rs = np.linalg.norm(from_dev(sd) - ws_) / np.linalg.norm(ws_)
    assert rs <= 1e-5, rs


@pytest.mark.parametrize("D", [128, 64])
def test_understated_key_norm_bound_still_correct(D):
    """key_norm_max far below the keys' norms.  Every key gets 20 u and every
    query u added, for one direction u of norm sqrt(D): the keys' norms grow to
    ~20 sqrt(D) while a bound of sqrt(D) is claimed, and every score gains the
    same 20 |u|^2 (softmax is unchanged by it, the bounded path overflows).
    The overflowing rows are detected by their row sums and recomputed on the
    running maximum; FULL (256- and 128-query shapes), RING in one launch,
    CHUNK_HYBRID and ROLLING all match the oracle."""
    H = 8
    pairs = (22, 21, 21) if D == 128 else (12, 10, 10)
    log(f"understated key_norm_max: D={D}")
    for L in (16347, 9001):
        grid = (1, 1, L)
        q, k, v = (raw((1, L, H, D), 320 + s + L) for s in range(3))
        qr, kr = V.vdit_rope_qk(to_dev(q), to_dev(k), V.make_grid(*grid, pairs))
        u = np.random.default_rng(330).standard_normal(D)
        u = torch.from_numpy(u * math.sqrt(D) / np.linalg.norm(u)).to(qr.dtype).cuda()
        qr.add_(u)
        kr.add_(20.0 * u)  # rounded to bf16; the oracle gets these values
        vd = to_dev(v)
        knm = math.sqrt(D)
        o, lse = V.vdit_attn_fwd(qr, kr, vd, key_norm_max=knm)
        kc, vc = [kr[:, :4000], kr[:, 4000:]], [vd[:, :4000], vd[:, 4000:]]
        r, rl = V.vdit_attn_fwd(qr, mode="ring", k_chunks=kc, v_chunks=vc, key_norm_max=knm)
        torch.cuda.synchronize()
        q64, k64 = from_dev(qr), from_dev(kr)
        rows = np.unique(np.concatenate([WL.sample_rows(L, 96, seed=L), [0, L - 1]]))
        wo, wl = O.attention(q64[:, rows], k64, v.values)
        check(from_dev(o)[:, rows], wo, "bf16", f"O FULL L={L} (sampled rows)")
        check_lse(from_dev(lse)[:, :, rows], wl, "bf16", f"LSE FULL L={L}")
        check(from_dev(r)[:, rows], wo, "bf16", f"O RING L={L} (sampled rows)")
        check_lse(from_dev(rl)[:, :, rows], wl, "bf16", f"LSE RING L={L}")
    # chunk hybrid (its own kernel instance): chunks of 1170, the last one
    # 811 tokens, whose last 128-query block has 43 queries (three wavefronts
    # without queries take the loads-and-barriers loop, in both passes)
    C = 1170
    sd = torch.zeros((1, H, D, D), device="cuda"); zd = torch.zeros((1, H, D), device="cuda")
    hq, hl = V.vdit_attn_fwd(qr, kr, vd, mode="hybrid", chunk_tokens=C, state_s=sd, state_z=zd, key_norm_max=knm)
    torch.cuda.synchronize()
    o_s, l_s, o_l, l_l = O.hybrid_partials(q64, k64, v.values, C)
    wo, wl = O.lse_merge(o_s, l_s, o_l, l_l)
    check(hq, wo, "bf16", "O HYBRID (all rows)")
    check_lse(hl, wl, "bf16", "LSE HYBRID")
    # rolling: 3 slots of 3000 tokens, frame 4
    kcache = kr[:, :9000].reshape(1, 3, 3000, H, D).contiguous()
    vcache = vd[:, :9000].reshape(1, 3, 3000, H, D).contiguous()
    qf = qr[:, :3000].contiguous()
    f, fl = V.vdit_attn_fwd(qf, mode="rolling", k_cache=kcache, v_cache=vcache, frame=4, key_norm_max=knm)
    torch.cuda.synchronize()
    rows = WL.sample_rows(3000, 64, seed=5)
    wo, wl = O.attention(q64[:, rows], k64[:, :9000], v.values[:, :9000])
    check(from_dev(f)[:, rows], wo, "bf16", "O ROLLING (sampled rows)")
    check_lse(from_dev(fl)[:, :, rows], wl, "bf16", "LSE ROLLING")
