"""Pins of the fp64 oracle against things other than itself.

Each test checks the oracle against a closed form, an invariant the pages
state, brute force on tiny inputs or an independent library routine, chosen
so that a plausible slip (a dropped term, a wrong sign or index, a transposed
operand, a wrong chunk boundary) fails at least one of them.  CPU only.
"""
import math
import os

import numpy as np
import pytest
import torch

import oracle as O
import workloads as WL

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
RNG = np.random.default_rng


def sdpa64(q, k, v, scale=None, mask=None):
    """torch float64 CPU scaled_dot_product_attention on [B,L,H,D] arrays."""
    tq = torch.from_numpy(np.ascontiguousarray(np.transpose(q, (0, 2, 1, 3))))
    tk = torch.from_numpy(np.ascontiguousarray(np.transpose(k, (0, 2, 1, 3))))
    tv = torch.from_numpy(np.ascontiguousarray(np.transpose(v, (0, 2, 1, 3))))
    m = None if mask is None else torch.from_numpy(mask)
    out = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=m, scale=scale)
    return np.transpose(out.numpy(), (0, 2, 1, 3))


# ------------------------------------------------------------- positions --

def test_grid_positions_t_major():
    t, h, w = O.grid_positions(72, (3, 4, 6))
    assert (t[0], h[0], w[0]) == (0, 0, 0)
    assert (t[1], h[1], w[1]) == (0, 0, 1)
    assert (t[6], h[6], w[6]) == (0, 1, 0)
    assert (t[24], h[24], w[24]) == (1, 0, 0)
    assert (t[71], h[71], w[71]) == (2, 3, 5)
    t2, h2, w2 = O.grid_positions(3, (3, 4, 6), token0=30, t_offset=5)
    assert list(t2) == [6, 6, 6] and list(h2) == [1, 1, 1] and list(w2) == [0, 1, 2]


# --------------------------------------------------------------- RMSNorm --

def test_rmsnorm_closed_form_values():
    # x = (3, 4): mean square 12.5 -> y = x / sqrt(12.5)
    y = O.rmsnorm(np.array([3.0, 4.0]), eps=0.0)
    assert np.allclose(y, [3 / math.sqrt(12.5), 4 / math.sqrt(12.5)], rtol=0, atol=1e-15)
    # eps enters under the root: x = (1, 1), eps = 1 -> 1/sqrt(2)
    y = O.rmsnorm(np.array([1.0, 1.0]), eps=1.0)
    assert np.allclose(y, [2 ** -0.5] * 2, atol=1e-15)
    # gain multiplies per channel
    y = O.rmsnorm(np.array([3.0, 4.0]), eps=0.0, gain=np.array([2.0, -1.0]))
    assert np.allclose(y, [6 / math.sqrt(12.5), -4 / math.sqrt(12.5)], atol=1e-15)


def test_rmsnorm_output_rms_and_scale_invariance():
    x = RNG(1).standard_normal((5, 7, 3, 64)) * 3.0
    eps = 1e-6
    y = O.rmsnorm(x, eps)
    ms = np.mean(x * x, axis=-1)
    rms_out = np.sqrt(np.mean(y * y, axis=-1))
    assert np.allclose(rms_out, np.sqrt(ms / (ms + eps)), rtol=1e-12)
    assert np.allclose(O.rmsnorm(x * 17.0, 0.0), O.rmsnorm(x, 0.0), rtol=1e-12)
    # per (token, head): normalising one head does not depend on another
    x2 = x.copy(); x2[:, :, 1, :] *= 100.0
    assert np.allclose(O.rmsnorm(x2, 0.0)[:, :, 0], O.rmsnorm(x, 0.0)[:, :, 0], rtol=1e-12)


# ------------------------------------------------------------------ RoPE --

def _read_rope_golden():
    cases = []
    with open(os.path.join(GOLDEN, "rope_closed_form.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            pairs, theta, pos, x, y = [s.strip() for s in line.split("|")]
            cases.append((tuple(int(v) for v in pairs.split()), float(theta),
                          tuple(int(v) for v in pos.split()),
                          np.array([float(v) for v in x.split()]),
                          np.array([float(v) for v in y.split()])))
    return cases


def test_rope_matches_hand_derived_golden():
    for pairs, theta, (t, h, w), x, y in _read_rope_golden():
        alpha = O.rope_angles(np.array([t]), np.array([h]), np.array([w]), pairs, theta)
        got = O.rope_rotate(x.reshape(1, 1, 1, 8), alpha).reshape(8)
        assert np.allclose(got, y, rtol=0, atol=1e-14), (pairs, got, y)


def test_rope_identity_at_origin_and_pair_norms():
    x = RNG(2).standard_normal((1, 72, 2, 64))
    alpha = O.rope_angles(*O.grid_positions(72, (3, 4, 6)), (12, 10, 10))
    y = O.rope_rotate(x, alpha)
    assert np.array_equal(y[:, 0], x[:, 0])          # token 0 sits at (0,0,0)
    n_in = x[..., 0::2] ** 2 + x[..., 1::2] ** 2
    n_out = y[..., 0::2] ** 2 + y[..., 1::2] ** 2
    assert np.allclose(n_in, n_out, rtol=1e-12)


def test_rope_reduces_to_textbook_1d_rope():
    # With T = H = 1 only the w block rotates; it must equal RoFormer's 1D
    # rotary embedding of dimension d = 2 P_w: multiply x_{2i} + i x_{2i+1} by
    # exp(i * w * 10000^(-2i/d)).
    Pt, Ph, Pw = 3, 2, 5
    D = 2 * (Pt + Ph + Pw)
    x = RNG(3).standard_normal((1, 9, 1, D))
    t, h, w = O.grid_positions(9, (1, 1, 9))
    y = O.rope_rotate(x, O.rope_angles(t, h, w, (Pt, Ph, Pw)))
    assert np.array_equal(y[..., : 2 * (Pt + Ph)], x[..., : 2 * (Pt + Ph)])
    d = 2 * Pw
    xc = x[0, :, 0, 2 * (Pt + Ph)::2] + 1j * x[0, :, 0, 2 * (Pt + Ph) + 1::2]
    freqs = np.array([10000.0 ** (-2 * i / d) for i in range(Pw)])
    yc = xc * np.exp(1j * np.outer(np.arange(9), freqs))
    got = y[0, :, 0, 2 * (Pt + Ph)::2] + 1j * y[0, :, 0, 2 * (Pt + Ph) + 1::2]
    assert np.allclose(got, yc, rtol=0, atol=1e-13)


@pytest.mark.parametrize("axis", [0, 1, 2])
def test_rope_relative_position_invariance(axis):
    # Shifting every t (or h, or w) by one constant leaves q.k unchanged:
    # R(a)^T R(b) = R(b - a) for each pair.
    L, H, D = 40, 2, 64
    pairs = (12, 10, 10)
    r = RNG(4 + axis)
    q = r.standard_normal((1, L, H, D)); k = r.standard_normal((1, L, H, D))
    pos = [r.integers(0, 9, L) for _ in range(3)]
    a0 = O.rope_angles(*pos, pairs)
    pos[axis] = pos[axis] + 13
    a1 = O.rope_angles(*pos, pairs)
    s0 = np.einsum("blhd,bmhd->bhlm", O.rope_rotate(q, a0), O.rope_rotate(k, a0))
    s1 = np.einsum("blhd,bmhd->bhlm", O.rope_rotate(q, a1), O.rope_rotate(k, a1))
    assert np.allclose(s0, s1, rtol=1e-11, atol=1e-11)
    # ... and a shift of q alone does change the scores (the pin is not vacuous)
    s2 = np.einsum("blhd,bmhd->bhlm", O.rope_rotate(q, a1), O.rope_rotate(k, a0))
    assert not np.allclose(s0, s2, atol=1e-3)


def test_rope_blockdiag_matrix_brute_force():
    # Brute force: build the explicit D x D block-diagonal rotation for one token
    # from its (t, h, w) position, axis by axis, and apply it as a matrix.
    pairs, theta = (3, 3, 2), 500.0
    D = 16
    x = RNG(7).standard_normal(D)
    t, h, w = 4, 1, 3
    M = np.zeros((D, D))
    p = 0
    for pos, Pa in ((t, pairs[0]), (h, pairs[1]), (w, pairs[2])):
        for j in range(Pa):
            a = pos * theta ** (-2.0 * j / (2 * Pa))
            M[2 * p, 2 * p] = math.cos(a); M[2 * p, 2 * p + 1] = -math.sin(a)
            M[2 * p + 1, 2 * p] = math.sin(a); M[2 * p + 1, 2 * p + 1] = math.cos(a)
            p += 1
    want = M @ x
    got = O.rope_rotate(x.reshape(1, 1, 1, D),
                        O.rope_angles(np.array([t]), np.array([h]), np.array([w]), pairs, theta))
    assert np.allclose(got.reshape(D), want, atol=1e-14)


def test_rope_qk_norm_then_rotate_and_v_untouched():
    q = RNG(8).standard_normal((1, 24, 2, 64)) * 5
    k = RNG(9).standard_normal((1, 24, 1, 64)) * 0.1
    qo, ko = O.rope_qk(q, k, (2, 3, 4), (12, 10, 10), eps=1e-6)
    # RMS of every (token, head) row is ~1 after norm, and rotation preserves it
    assert np.allclose(np.sqrt(np.mean(qo ** 2, -1)), 1.0, atol=1e-6)
    assert np.allclose(np.sqrt(np.mean(ko ** 2, -1)), 1.0, atol=1e-4)
    qn, kn = O.rope_qk(q, k, (2, 3, 4), (12, 10, 10), norm=False)
    assert np.allclose(np.sqrt(np.mean(qn ** 2, -1)), np.sqrt(np.mean(q ** 2, -1)))


# ------------------------------------------------------------- attention --

def test_attention_brute_force_loops():
    r = RNG(10)
    B, Lq, Lk, Hq, Hk, D = 1, 4, 5, 2, 1, 3
    q = r.standard_normal((B, Lq, Hq, D)); k = r.standard_normal((B, Lk, Hk, D))
    v = r.standard_normal((B, Lk, Hk, D))
    scale = 0.7
    o, lse = O.attention(q, k, v, scale)
    for h in range(Hq):
        for i in range(Lq):
            s = [scale * math.fsum(q[0, i, h, d] * k[0, j, 0, d] for d in range(D)) for j in range(Lk)]
            e = [math.exp(x) for x in s]
            z = math.fsum(e)
            assert abs(lse[0, h, i] - math.log(z)) < 1e-12
            for d in range(D):
                want = math.fsum(e[j] * v[0, j, 0, d] for j in range(Lk)) / z
                assert abs(o[0, i, h, d] - want) < 1e-12


@pytest.mark.parametrize("Hq,Hk", [(2, 2), (4, 2), (6, 3)])
def test_attention_matches_torch_sdpa_f64(Hq, Hk):
    r = RNG(11)
    q = r.standard_normal((2, 33, Hq, 16)); k = r.standard_normal((2, 47, Hk, 16))
    v = r.standard_normal((2, 47, Hk, 16))
    o, lse = O.attention(q, k, v)
    rep = Hq // Hk
    want = sdpa64(q, np.repeat(k, rep, axis=2), np.repeat(v, rep, axis=2))
    assert np.allclose(o, want, atol=1e-12)
    from scipy.special import logsumexp
    s = np.einsum("bihd,bjhd->bhij", q, np.repeat(k, rep, axis=2)) / 4.0
    assert np.allclose(lse, logsumexp(s, axis=-1), atol=1e-12)


def test_attention_probs_brute_force_and_against_attention():
    # The softmax weight matrix: rows sum to one, each entry is
    # e^{s_ij} / sum_k e^{s_ik} by loops (scale and GQA head map included),
    # P V is attention's output and ln of the row normaliser its LSE.
    r = RNG(15)
    B, Lq, Lk, Hq, Hk, D, scale = 2, 5, 7, 4, 2, 6, 0.45
    q = r.standard_normal((B, Lq, Hq, D)); k = r.standard_normal((B, Lk, Hk, D))
    v = r.standard_normal((B, Lk, Hk, D))
    P = O.attention_probs(q, k, scale)
    assert P.shape == (B, Hq, Lq, Lk)
    assert np.allclose(P.sum(-1), 1.0, atol=1e-14) and (P >= 0).all()
    for b in range(B):
        for h in range(Hq):
            kh = h // (Hq // Hk)
            for i in range(Lq):
                e = [math.exp(scale * math.fsum(q[b, i, h, d] * k[b, j, kh, d] for d in range(D))) for j in range(Lk)]
                z = math.fsum(e)
                for j in range(Lk):
                    assert abs(P[b, h, i, j] - e[j] / z) < 1e-14
    o, lse = O.attention(q, k, v, scale)
    rep = Hq // Hk
    pv = np.einsum("bhij,bjhd->bihd", P, np.repeat(v, rep, axis=2))
    assert np.allclose(pv, o, atol=1e-13)
    # a score shifted by a constant per row leaves P unchanged: the LSE is the
    # only row-dependent normaliser, so ln P_ij = s_ij - LSE_i
    s = scale * np.einsum("bihd,bjhd->bhij", q, np.repeat(k, rep, axis=2))
    assert np.allclose(np.log(P), s - lse[..., None], atol=1e-12)


def test_attention_special_cases():
    r = RNG(12)
    q = r.standard_normal((1, 6, 1, 8))
    # identical keys -> mean of V
    k = np.repeat(r.standard_normal((1, 1, 1, 8)), 5, axis=1)
    v = r.standard_normal((1, 5, 1, 8))
    o, _ = O.attention(q, k, v)
    assert np.allclose(o, v.mean(axis=1, keepdims=True).repeat(6, axis=1), atol=1e-14)
    # one key -> that value, LSE = its score
    o, lse = O.attention(q, k[:, :1], v[:, :1])
    assert np.allclose(o, np.repeat(v[:, :1], 6, axis=1))
    assert np.allclose(lse[0, 0], (q[0, :, 0] @ k[0, 0, 0]) / math.sqrt(8))
    # constant value rows -> that row
    vc = np.repeat(r.standard_normal((1, 1, 1, 8)), 9, axis=1)
    o, _ = O.attention(q, r.standard_normal((1, 9, 1, 8)), vc)
    assert np.allclose(o, np.repeat(vc[:, :1], 6, axis=1), atol=1e-14)
    # empty key set -> O = 0, LSE = -inf
    o, lse = O.attention(q, np.zeros((1, 0, 1, 8)), np.zeros((1, 0, 1, 8)))
    assert (o == 0).all() and np.isneginf(lse).all()


def test_attention_key_permutation_invariance():
    r = RNG(13)
    q = r.standard_normal((1, 7, 2, 16)); k = r.standard_normal((1, 30, 2, 16))
    v = r.standard_normal((1, 30, 2, 16))
    perm = r.permutation(30)
    o1, l1 = O.attention(q, k, v); o2, l2 = O.attention(q, k[:, perm], v[:, perm])
    assert np.allclose(o1, o2, atol=1e-13) and np.allclose(l1, l2, atol=1e-13)


# ----------------------------------------------------------- merge, ring --

def test_merge_of_any_partition_equals_full():
    r = RNG(14)
    q = r.standard_normal((1, 11, 2, 16)); k = r.standard_normal((1, 40, 2, 16))
    v = r.standard_normal((1, 40, 2, 16))
    o_full, l_full = O.attention(q, k, v)
    for cuts in ([13], [5, 21, 33], [1, 2, 39]):
        bounds = [0] + cuts + [40]
        parts = [(k[:, a:b], v[:, a:b]) for a, b in zip(bounds[:-1], bounds[1:])]
        o, l = O.attention(q, *parts[0])
        for kc, vc in parts[1:]:
            o, l = O.lse_merge(o, l, *O.attention(q, kc, vc))
        assert np.allclose(o, o_full, atol=1e-13) and np.allclose(l, l_full, atol=1e-13)


def test_merge_commutative_associative_identity():
    r = RNG(15)
    parts = []
    for _ in range(3):
        parts.append((r.standard_normal((1, 5, 2, 8)), r.standard_normal((1, 2, 5))))
    a, b, c = parts
    ab = O.lse_merge(*a, *b); ba = O.lse_merge(*b, *a)
    assert np.allclose(ab[0], ba[0]) and np.allclose(ab[1], ba[1])
    l1 = O.lse_merge(*O.lse_merge(*a, *b), *c); l2 = O.lse_merge(*a, *O.lse_merge(*b, *c))
    assert np.allclose(l1[0], l2[0]) and np.allclose(l1[1], l2[1])
    empty = (np.zeros((1, 5, 2, 8)), np.full((1, 2, 5), -np.inf))
    ae = O.lse_merge(*a, *empty)
    assert np.allclose(ae[0], a[0]) and np.allclose(ae[1], a[1])
    ee = O.lse_merge(*empty, *empty)
    assert (ee[0] == 0).all() and np.isneginf(ee[1]).all()


def test_ring_equals_full_attention():
    # ReGenVC (USP paragraph): ring attention is exact up to reduction order.
    r = RNG(16)
    q = r.standard_normal((1, 20, 3, 16)); k = r.standard_normal((1, 48, 3, 16))
    v = r.standard_normal((1, 48, 3, 16))
    o_full, l_full = O.attention(q, k, v)
    o, l = O.ring_attention(q, [k[:, :24], k[:, 24:]], [v[:, :24], v[:, 24:]])
    assert np.allclose(o, o_full, atol=1e-13) and np.allclose(l, l_full, atol=1e-13)
    o, l = O.ring_attention(q, [k[:, 30:], k[:, :30]], [v[:, 30:], v[:, :30]])
    assert np.allclose(o, o_full, atol=1e-13)


# --------------------------------------------------------------- rolling --

def test_rolling_window_matches_page_statement():
    with open(os.path.join(GOLDEN, "window_pattern.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            W, fr, frames = [s.strip() for s in line.split("|")]
            assert list(O.rolling_window(int(fr), int(W))) == [int(x) for x in frames.split()]


def _roped_all(qf, kf, frame_grid, pairs, t_of_frame):
    F = qf.shape[0]
    qs, ks = [], []
    for u in range(F):
        a, b = O.rope_qk(qf[u][None], kf[u][None], frame_grid, pairs, t_offset=t_of_frame[u])
        qs.append(a); ks.append(b)
    return qs, ks


@pytest.mark.parametrize("W", [1, 2, 3, 6])
def test_rolling_equals_masked_brute_force(W):
    # FlashDecoder Sec. 3.3: the window pattern equals attention over all frames
    # with a mask admitting frames f0..f; here built with an explicit mask.
    F, grid, H, D, pairs = 5, (1, 2, 3), 2, 16, (2, 3, 3)
    L = 6
    r = RNG(20 + W)
    qf = r.standard_normal((F, L, H, D)); kf = r.standard_normal((F, L, H, D))
    vf = r.standard_normal((F, L, H, D))
    for f in range(F):
        f0 = max(0, f - W + 1)
        qs, ks = _roped_all(qf, kf, grid, pairs, [u - f0 for u in range(F)])
        K = np.concatenate(ks, axis=1); V = np.concatenate([vf[u][None] for u in range(F)], axis=1)
        frame_of_key = np.repeat(np.arange(F), L)
        allowed = (frame_of_key >= f0) & (frame_of_key <= f)
        mask = np.where(allowed, 0.0, -np.inf)[None, None, None, :].repeat(L, axis=2)
        want = sdpa64(qs[f], K, V, mask=mask)
        got, _ = O.rolling_frame(qf, kf, vf, f, W, grid, pairs)
        assert np.allclose(got, want, atol=1e-12), (W, f)


def test_rolling_window_relative_equals_absolute_positions():
    # Window-relative t (FlashDecoder Sec. 4, "Long Video Decoding") and absolute t
    # give the same scores: RoPE depends on position differences only.
    F, grid, H, D, pairs, W = 6, (1, 2, 2), 1, 16, (3, 3, 2), 3
    r = RNG(30)
    qf = r.standard_normal((F, 4, H, D)); kf = r.standard_normal((F, 4, H, D))
    vf = r.standard_normal((F, 4, H, D))
    f = 5
    qs, ks = _roped_all(qf, kf, grid, pairs, list(range(F)))  # absolute t = u
    win = list(O.rolling_window(f, W))
    want, _ = O.attention(qs[f], np.concatenate([ks[u] for u in win], 1),
                          np.concatenate([vf[u][None] for u in win], 1))
    got, _ = O.rolling_frame(qf, kf, vf, f, W, grid, pairs)
    assert np.allclose(got, want, atol=1e-12)


def test_rolling_degenerate_windows():
    F, grid, H, D, pairs = 4, (1, 2, 2), 1, 8, (2, 1, 1)
    r = RNG(31)
    qf = r.standard_normal((F, 4, H, D)); kf = r.standard_normal((F, 4, H, D))
    vf = r.standard_normal((F, 4, H, D))
    # W = 1: per-frame attention at t = 0
    for f in range(F):
        a, b = O.rope_qk(qf[f][None], kf[f][None], grid, pairs)
        want, _ = O.attention(a, b, vf[f][None])
        got, _ = O.rolling_frame(qf, kf, vf, f, 1, grid, pairs)
        assert np.allclose(got, want, atol=1e-13)
    # W >= F: block-causal over all earlier frames with absolute t
    qs, ks = _roped_all(qf, kf, grid, pairs, list(range(F)))
    for f in range(F):
        want, _ = O.attention(qs[f], np.concatenate(ks[: f + 1], 1),
                              np.concatenate([vf[u][None] for u in range(f + 1)], 1))
        got, _ = O.rolling_frame(qf, kf, vf, f, 10, grid, pairs)
        assert np.allclose(got, want, atol=1e-12)


def _rms_rows(x, eps=1e-6):
    # RMSNorm written out from its definition: x / sqrt(mean over the head dim of x^2 + eps)
    return x / np.sqrt((x * x).mean(axis=-1, keepdims=True) + eps)


@pytest.mark.parametrize("W", [1, 2, 3])
def test_rolling_kv_norm_gqa_equals_masked_brute_force(W):
    # FlashDecoder Sec. 3.2: GQA and KV-norm (keys and values normalised inside
    # attention, queries not); Sec. 3.3: the window as a frame mask.  Expected
    # values: q rotated without a norm, k normalised then rotated, v normalised,
    # KV heads repeated per query group by hand, one masked softmax over all frames.
    F, grid, Hq, Hk, D, pairs = 4, (1, 2, 3), 6, 2, 16, (2, 3, 3)
    L = 6
    r = RNG(40 + W)
    qf = 3.0 * r.standard_normal((F, L, Hq, D)); kf = 2.0 * r.standard_normal((F, L, Hk, D))
    vf = 5.0 * r.standard_normal((F, L, Hk, D))
    for f in range(F):
        f0 = max(0, f - W + 1)
        qs, ks = [], []
        for u in range(F):
            a, _ = O.rope_qk(qf[u][None], qf[u][None], grid, pairs, t_offset=u - f0, norm=False)
            _, b = O.rope_qk(kf[u][None], _rms_rows(kf[u][None]), grid, pairs, t_offset=u - f0, norm=False)
            qs.append(a); ks.append(b)
        K = np.repeat(np.concatenate(ks, axis=1), Hq // Hk, axis=2)
        Vv = np.repeat(np.concatenate([_rms_rows(vf[u][None]) for u in range(F)], axis=1), Hq // Hk, axis=2)
        frame_of_key = np.repeat(np.arange(F), L)
        allowed = (frame_of_key >= f0) & (frame_of_key <= f)
        mask = np.where(allowed, 0.0, -np.inf)[None, None, None, :].repeat(L, axis=2)
        want = sdpa64(qs[f], K, Vv, mask=mask)
        got, _ = O.rolling_frame(qf, kf, vf, f, W, grid, pairs, kv_norm=True)
        assert np.allclose(got, want, atol=1e-12), (W, f)


def test_rolling_kv_norm_scale_behaviour():
    # With KV-norm, scaling a frame's keys or values by a positive factor leaves
    # the output unchanged (up to eps); scaling the queries sharpens the softmax
    # and changes it.  A slip that normalises q, or skips v, fails here.
    F, grid, H, D, pairs, W, f = 3, (1, 2, 2), 2, 16, (3, 3, 2), 2, 2
    r = RNG(45)
    qf = r.standard_normal((F, 4, H, D)); kf = r.standard_normal((F, 4, H, D))
    vf = r.standard_normal((F, 4, H, D))
    base, _ = O.rolling_frame(qf, kf, vf, f, W, grid, pairs, kv_norm=True, eps=0.0)
    k2 = kf.copy(); k2[1] *= 7.0
    v2 = vf.copy(); v2[2] *= 0.25
    got_k, _ = O.rolling_frame(qf, k2, vf, f, W, grid, pairs, kv_norm=True, eps=0.0)
    got_v, _ = O.rolling_frame(qf, kf, v2, f, W, grid, pairs, kv_norm=True, eps=0.0)
    assert np.allclose(got_k, base, atol=1e-13) and np.allclose(got_v, base, atol=1e-13)
    q2 = qf.copy(); q2[f] *= 3.0
    got_q, _ = O.rolling_frame(q2, kf, vf, f, W, grid, pairs, kv_norm=True, eps=0.0)
    assert np.abs(got_q - base).max() > 1e-3
    # every output row of a KV-normed window has RMS over D at most 1 (a convex
    # combination of unit-RMS value rows)
    rms = np.sqrt((base * base).mean(axis=-1))
    assert (rms <= 1.0 + 1e-12).all()


@pytest.mark.parametrize("W", [1, 2])
def test_rolling_steps_of_subframes_equal_global_grid(W):
    # FlashDecoder Sec. 3.4, Step 2: a refinement step carries r_t sub-frames of
    # one latent frame and the window spans r_t * W sub-frames.  Expected values:
    # rotate every token once at its absolute position on the global grid
    # (r_t * F sub-frames), then a masked softmax admitting the keys of steps
    # f0..f.  RoPE's relative invariance makes the window-relative positions of
    # the oracle give the same scores.
    F, rt, Hh, Ww, H, D, pairs = 4, 3, 2, 2, 2, 16, (3, 3, 2)
    Ls = rt * Hh * Ww
    r = RNG(50 + W)
    qf = r.standard_normal((F, Ls, H, D)); kf = r.standard_normal((F, Ls, H, D))
    vf = r.standard_normal((F, Ls, H, D))
    qa, ka = O.rope_qk(qf.reshape(1, F * Ls, H, D), kf.reshape(1, F * Ls, H, D), (rt * F, Hh, Ww), pairs)
    Vv = vf.reshape(1, F * Ls, H, D)
    step_of_key = np.repeat(np.arange(F), Ls)
    for f in range(F):
        f0 = max(0, f - W + 1)
        allowed = (step_of_key >= f0) & (step_of_key <= f)
        mask = np.where(allowed, 0.0, -np.inf)[None, None, None, :].repeat(Ls, axis=2)
        want = sdpa64(qa[:, f * Ls:(f + 1) * Ls], ka, Vv, mask=mask)
        got, _ = O.rolling_frame(qf, kf, vf, f, W, (rt, Hh, Ww), pairs)
        assert np.allclose(got, want, atol=1e-12), (W, f)


# ---------------------------------------------------------------- hybrid --

def test_phi_is_elu_plus_one():
    x = np.array([-3.0, -1.0, 0.0, 0.5, 2.0])
    assert np.allclose(O.phi(x), [math.exp(-3), math.exp(-1), 1.0, 1.5, 3.0], atol=1e-15)
    t = torch.nn.functional.elu(torch.linspace(-5, 5, 101, dtype=torch.float64)) + 1
    assert np.allclose(O.phi(np.linspace(-5, 5, 101)), t.numpy(), atol=1e-15)


def _elu1(x):
    return x + 1 if x > 0 else math.exp(x)


def _hybrid_brute(q, k, v, C, scale, overlap=0, fmap_q=_elu1, fmap_k=_elu1):
    # Full L x L weight matrix by loops: key in the query's chunk or in the
    # `overlap` tokens before that chunk -> e^{s_ij}; any earlier key ->
    # phi_q(q_i).phi_k(k_j); later key -> 0.  O = W V / W 1.
    B, L, H, D = q.shape
    out = np.zeros_like(q)
    for h in range(H):
        for i in range(L):
            start = (i // C) * C
            wts = []
            for j in range(L):
                if start - overlap <= j < start + C:
                    s = scale * math.fsum(q[0, i, h, d] * k[0, j, h, d] for d in range(D))
                    wts.append(math.exp(s))
                elif j < start - overlap:
                    fq = [fmap_q(q[0, i, h, d]) for d in range(D)]
                    fk = [fmap_k(k[0, j, h, d]) for d in range(D)]
                    wts.append(math.fsum(a * b for a, b in zip(fq, fk)))
                else:
                    wts.append(0.0)
            den = math.fsum(wts)
            for d in range(D):
                out[0, i, h, d] = math.fsum(wts[j] * v[0, j, h, d] for j in range(L)) / den
    return out


# Degree-3 feature maps (MobileWan review, ledger: polynomial phi_q, phi_k of
# degree 3, Appendix A.3.1).  Synthetic coefficients, positive on [-3, 3].
POLY = (1.0, 0.3, 0.05, 0.004, 0.8, -0.2, 0.06, 0.003)


def test_phi_poly_coefficient_order():
    # c0 + c1 x + c2 x^2 + c3 x^3 at hand-computed points
    assert O.phi_poly(np.array([2.0]), (1.0, 0.5, 0.25, 0.125))[0] == 4.0
    assert O.phi_poly(np.array([-2.0]), (1.0, 0.5, 0.25, 0.125))[0] == 0.0
    assert O.phi_poly(np.array([3.0]), (0.0, 0.0, 0.0, 1.0))[0] == 27.0
    assert O.phi_poly(np.array([3.0]), (0.0, 0.0, 1.0, 0.0))[0] == 9.0
    x = np.linspace(-4, 4, 33)
    assert np.allclose(O.phi_poly(x, POLY[4:]), np.polynomial.polynomial.polyval(x, POLY[4:]), atol=1e-14)


@pytest.mark.parametrize("overlap", [0, 3])
def test_hybrid_polynomial_phi_matches_brute_force(overlap):
    r = RNG(70 + overlap)
    q = r.standard_normal((1, 11, 2, 4)); k = r.standard_normal((1, 11, 2, 4))
    v = r.standard_normal((1, 11, 2, 4))
    fq = lambda x: float(np.polynomial.polynomial.polyval(x, POLY[:4]))
    fk = lambda x: float(np.polynomial.polynomial.polyval(x, POLY[4:]))
    want = _hybrid_brute(q, k, v, 4, 0.5, overlap, fq, fk)
    o_e, _, _, _ = O.hybrid_explicit(q, k, v, 4, 0.5, overlap=overlap, phi_coef=POLY)
    o_r, _, _, _ = O.hybrid_recurrent(q, k, v, 4, 0.5, overlap=overlap, phi_coef=POLY)
    assert np.allclose(o_e, want, atol=1e-12)
    assert np.allclose(o_r, want, atol=1e-12)
    # phi_q and phi_k are not interchangeable, and differ from elu + 1
    swapped = POLY[4:] + POLY[:4]
    o_s, _, _, _ = O.hybrid_explicit(q, k, v, 4, 0.5, overlap=overlap, phi_coef=swapped)
    o_elu, _, _, _ = O.hybrid_explicit(q, k, v, 4, 0.5, overlap=overlap)
    assert np.abs(o_s - want).max() > 1e-4 and np.abs(o_elu - want).max() > 1e-4


def test_hybrid_polynomial_phi_closed_forms():
    r = RNG(73)
    B, L, H, D, C = 1, 12, 2, 8, 4
    q = r.standard_normal((B, L, H, D)); k = r.standard_normal((B, L, H, D))
    v = r.standard_normal((B, L, H, D))
    # constant maps phi_q = a, phi_k = b: every earlier key weighs D a b, so the
    # linear partial is the mean of the earlier values and its LSE ln(n D a b)
    a, b = 0.7, 1.3
    _, _, o_l, l_l = O.hybrid_partials(q, k, v, C, phi_coef=(a, 0, 0, 0, b, 0, 0, 0))
    for c0 in range(C, L, C):
        assert np.allclose(o_l[:, c0:c0 + C], v[:, :c0].mean(axis=1, keepdims=True), atol=1e-13)
        assert np.allclose(l_l[:, :, c0:c0 + C], math.log(c0 * D * a * b), atol=1e-13)
    # pure cubes: phi_q(q).phi_k(k) = sum_d q_d^3 k_d^3
    _, _, o_l, l_l = O.hybrid_partials(q, k, v, C, phi_coef=(0, 0, 0, 1, 0, 0, 0, 1))
    i, h, c0 = 9, 1, 8
    w = [math.fsum(q[0, i, h, d] ** 3 * k[0, j, h, d] ** 3 for d in range(D)) for j in range(c0)]
    den = math.fsum(w)
    if den > 0:
        assert abs(l_l[0, h, i] - math.log(den)) < 1e-12
        for d in range(D):
            assert abs(o_l[0, i, h, d] - math.fsum(w[j] * v[0, j, h, d] for j in range(c0)) / den) < 1e-12
    else:  # a normaliser that is not positive drops the linear partial
        assert np.isneginf(l_l[0, h, i]) and not o_l[0, i, h].any()


def test_hybrid_polynomial_recurrent_equals_explicit_and_state():
    r = RNG(74)
    B, L, Hq, Hk, D, C, Ov = 2, 29, 4, 2, 8, 7, 3
    q = r.standard_normal((B, L, Hq, D)); k = r.standard_normal((B, L, Hk, D))
    v = r.standard_normal((B, L, Hk, D))
    s0 = r.standard_normal((B, Hk, D, D)) * 0.1; z0 = np.abs(r.standard_normal((B, Hk, D)))
    e = O.hybrid_explicit(q, k, v, C, s0=s0, z0=z0, overlap=Ov, phi_coef=POLY)
    rr = O.hybrid_recurrent(q, k, v, C, s0=s0, z0=z0, overlap=Ov, phi_coef=POLY)
    for x, y in zip(e, rr):
        assert np.allclose(x, y, atol=1e-11)
    s_want = s0.copy(); z_want = z0.copy()
    for bb in range(B):
        for h in range(Hk):
            for j in range(L - Ov):
                fk = np.polynomial.polynomial.polyval(k[bb, j, h], POLY[4:])
                s_want[bb, h] += np.outer(fk, v[bb, j, h])
                z_want[bb, h] += fk
    assert np.allclose(rr[2], s_want, atol=1e-11) and np.allclose(rr[3], z_want, atol=1e-11)


def test_hybrid_matches_brute_force_weight_matrix():
    r = RNG(40)
    q = r.standard_normal((1, 11, 2, 4)); k = r.standard_normal((1, 11, 2, 4))
    v = r.standard_normal((1, 11, 2, 4))
    want = _hybrid_brute(q, k, v, 4, 0.5)
    o_e, _, _, _ = O.hybrid_explicit(q, k, v, 4, 0.5)
    o_r, _, _, _ = O.hybrid_recurrent(q, k, v, 4, 0.5)
    assert np.allclose(o_e, want, atol=1e-12)
    assert np.allclose(o_r, want, atol=1e-12)


@pytest.mark.parametrize("overlap", [2, 5, 9])
def test_hybrid_overlap_matches_brute_force_weight_matrix(overlap):
    # MobileWan review, Appendix A.3.1 (ledger): the softmax window of a chunk
    # reaches T_o slices back; keys before the window go through the linear
    # term, each key exactly once.
    r = RNG(60 + overlap)
    q = r.standard_normal((1, 11, 2, 4)); k = r.standard_normal((1, 11, 2, 4))
    v = r.standard_normal((1, 11, 2, 4))
    want = _hybrid_brute(q, k, v, 4, 0.5, overlap)
    o_e, _, _, _ = O.hybrid_explicit(q, k, v, 4, 0.5, overlap=overlap)
    o_r, _, _, _ = O.hybrid_recurrent(q, k, v, 4, 0.5, overlap=overlap)
    assert np.allclose(o_e, want, atol=1e-12)
    assert np.allclose(o_r, want, atol=1e-12)
    if overlap:
        o_0, _, _, _ = O.hybrid_explicit(q, k, v, 4, 0.5)
        assert np.abs(o_0 - want).max() > 1e-3  # the overlap changes the result


def test_hybrid_overlap_recurrent_equals_explicit_and_state():
    r = RNG(62)
    B, L, Hq, Hk, D, C, Ov = 2, 37, 4, 2, 8, 9, 4
    q = r.standard_normal((B, L, Hq, D)); k = r.standard_normal((B, L, Hk, D))
    v = r.standard_normal((B, L, Hk, D))
    s0 = r.standard_normal((B, Hk, D, D)) * 0.1; z0 = np.abs(r.standard_normal((B, Hk, D)))
    e = O.hybrid_explicit(q, k, v, C, s0=s0, z0=z0, overlap=Ov)
    rr = O.hybrid_recurrent(q, k, v, C, s0=s0, z0=z0, overlap=Ov)
    for a, b in zip(e, rr):
        assert np.allclose(a, b, atol=1e-11)
    # final state: all keys but the last Ov, by loops
    fk = O.phi(k)
    s_want = s0.copy(); z_want = z0.copy()
    for b in range(B):
        for h in range(Hk):
            for j in range(L - Ov):
                s_want[b, h] += np.outer(fk[b, j, h], v[b, j, h])
                z_want[b, h] += fk[b, j, h]
    assert np.allclose(rr[2], s_want, atol=1e-11) and np.allclose(rr[3], z_want, atol=1e-11)


def test_hybrid_overlap_streaming_calls_with_context_equal_one_call():
    # Streaming with overlap: each call after the first passes the previous
    # call's last `overlap` keys/values as context ahead of its queries.
    r = RNG(63)
    L, C, Ov = 30, 6, 4
    q = r.standard_normal((1, L, 2, 8)); k = r.standard_normal((1, L, 2, 8))
    v = r.standard_normal((1, L, 2, 8))
    o, lse, s, z = O.hybrid_recurrent(q, k, v, C, overlap=Ov)
    outs, st, zt = [], None, None
    for a, b in ((0, 12), (12, 18), (18, 30)):
        c = min(Ov, a)
        oc, lc, st, zt = O.hybrid_explicit(q[:, a:b], k[:, a - c:b], v[:, a - c:b], C, s0=st, z0=zt,
                                           overlap=Ov, ctx=c)
        outs.append((oc, lc))
    assert np.allclose(np.concatenate([x[0] for x in outs], 1), o, atol=1e-12)
    assert np.allclose(np.concatenate([x[1] for x in outs], 2), lse, atol=1e-12)
    assert np.allclose(st, s, atol=1e-12) and np.allclose(zt, z, atol=1e-12)


def test_hybrid_overlap_covering_everything_is_block_causal_softmax():
    # With the window reaching back to the first key no linear term is left:
    # chunk-causal softmax attention (masked torch float64 SDPA).
    r = RNG(64)
    L, C = 14, 4
    q = r.standard_normal((1, L, 2, 8)); k = r.standard_normal((1, L, 2, 8))
    v = r.standard_normal((1, L, 2, 8))
    o, _, s, z = O.hybrid_explicit(q, k, v, C, overlap=L)
    chunk = np.arange(L) // C
    mask = np.where(chunk[None, :] <= chunk[:, None], 0.0, -np.inf)[None, None]
    assert np.allclose(o, sdpa64(q, k, v, mask=mask), atol=1e-12)
    assert not s.any() and not z.any()


def test_hybrid_recurrent_equals_explicit_and_state():
    # MobileWan review: the RNN form is the standard equivalence of causal linear attention.
    r = RNG(41)
    B, L, Hq, Hk, D, C = 2, 37, 4, 2, 8, 9
    q = r.standard_normal((B, L, Hq, D)); k = r.standard_normal((B, L, Hk, D))
    v = r.standard_normal((B, L, Hk, D))
    s0 = r.standard_normal((B, Hk, D, D)) * 0.1; z0 = np.abs(r.standard_normal((B, Hk, D)))
    e = O.hybrid_explicit(q, k, v, C, s0=s0, z0=z0)
    rr = O.hybrid_recurrent(q, k, v, C, s0=s0, z0=z0)
    for a, b in zip(e, rr):
        assert np.allclose(a, b, atol=1e-11)
    # final state = s0 + sum_j phi(k_j) v_j^T, by loops
    fk = O.phi(k)
    s_want = s0.copy()
    for b in range(B):
        for h in range(Hk):
            for j in range(L):
                s_want[b, h] += np.outer(fk[b, j, h], v[b, j, h])
    assert np.allclose(rr[2], s_want, atol=1e-11)
    assert np.allclose(rr[3], z0 + fk.sum(axis=1), atol=1e-11)


def test_hybrid_special_cases():
    r = RNG(42)
    q = r.standard_normal((1, 20, 2, 8)); k = r.standard_normal((1, 20, 2, 8))
    v = r.standard_normal((1, 20, 2, 8))
    # chunk 0 is pure softmax over its own chunk
    o, lse, _, _ = O.hybrid_recurrent(q, k, v, 6)
    o0, l0 = O.attention(q[:, :6], k[:, :6], v[:, :6])
    assert np.allclose(o[:, :6], o0, atol=1e-13) and np.allclose(lse[:, :, :6], l0, atol=1e-13)
    # one chunk covering everything is full attention
    o, lse, _, _ = O.hybrid_recurrent(q, k, v, 20)
    of, lf = O.attention(q, k, v)
    assert np.allclose(o, of, atol=1e-13) and np.allclose(lse, lf, atol=1e-13)
    o, _, _, _ = O.hybrid_explicit(q, k, v, 100)
    assert np.allclose(o, of, atol=1e-13)


def test_hybrid_split_calls_equal_one_call():
    # Streaming: two calls (split on a chunk boundary) carrying the state equal one call.
    r = RNG(43)
    q = r.standard_normal((1, 24, 2, 8)); k = r.standard_normal((1, 24, 2, 8))
    v = r.standard_normal((1, 24, 2, 8))
    o, lse, s, z = O.hybrid_recurrent(q, k, v, 6)
    o1, l1, s1, z1 = O.hybrid_recurrent(q[:, :12], k[:, :12], v[:, :12], 6)
    o2, l2, s2, z2 = O.hybrid_recurrent(q[:, 12:], k[:, 12:], v[:, 12:], 6, s0=s1, z0=z1)
    assert np.allclose(np.concatenate([o1, o2], 1), o, atol=1e-12)
    assert np.allclose(s2, s, atol=1e-12) and np.allclose(z2, z, atol=1e-12)


def test_hybrid_partials_merge_to_output():
    r = RNG(44)
    q = r.standard_normal((1, 15, 2, 8)); k = r.standard_normal((1, 15, 2, 8))
    v = r.standard_normal((1, 15, 2, 8))
    o, lse, _, _ = O.hybrid_explicit(q, k, v, 4)
    o_s, l_s, o_l, l_l = O.hybrid_partials(q, k, v, 4)
    m, lm = O.lse_merge(o_s, l_s, o_l, l_l)
    assert np.allclose(m, o, atol=1e-12) and np.allclose(lm, lse, atol=1e-12)
    assert np.isneginf(l_l[:, :, :4]).all() and np.isfinite(l_l[:, :, 4:]).all()
    # overlap 5: chunk 1's window reaches key 0 (no linear term), chunk 2's starts at key 3
    o, lse, _, _ = O.hybrid_explicit(q, k, v, 4, overlap=5)
    o_s, l_s, o_l, l_l = O.hybrid_partials(q, k, v, 4, overlap=5)
    m, lm = O.lse_merge(o_s, l_s, o_l, l_l)
    assert np.allclose(m, o, atol=1e-12) and np.allclose(lm, lse, atol=1e-12)
    assert np.isneginf(l_l[:, :, :8]).all() and np.isfinite(l_l[:, :, 8:]).all()


# ------------------------------------------------------------- workloads --

def test_bf16_rounding_matches_torch():
    x = RNG(50).standard_normal(10000).astype(np.float32)
    x[:4] = [1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -1.0 - 2 ** -8, 3.0]   # ties
    got = WL.bf16_bits_to_f64(WL.f32_to_bf16_bits(x))
    want = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(got, want)


def test_workload_shapes_and_flop_counts():
    w2 = WL.WORKLOADS[2]
    assert w2.tokens == 32760 and sum(w2.pairs) * 2 == w2.head_dim
    assert abs(WL.flops_full(32760, 32760, 12, 128) / 1e12 - 6.5938) < 1e-4
    w3 = WL.WORKLOADS[3]
    assert abs(2 * WL.flops_full(15600, 15600, 10, 128) / 1e12 - 2.4920) < 1e-4
    w4 = WL.WORKLOADS[4]
    assert w4.tokens == 2040 and sum(w4.pairs) * 2 == w4.head_dim
    w5 = WL.WORKLOADS[5]
    assert w5.tokens == 12090 and w5.chunk_tokens == 3 * 15 * 26
    assert abs(WL.hybrid_flops(w5) / 1e12 - 0.1701) < 1e-4  # chunk-local softmax work
    w8 = WL.WORKLOADS[8]
    assert w8.chunk_tokens == 4 * 15 * 26 and w8.overlap_tokens == 2 * 15 * 26  # T_c = 4, T_o = 2
    # FlashDecoder-XL (Table 5: width 1536, 24 heads, 3 KV groups; W_frm = 2),
    # 720p latents at spatial compression 16: 45 x 80 tokens per frame
    w6, w7 = WL.WORKLOADS[6], WL.WORKLOADS[7]
    assert w6.tokens == 3600 and w6.heads * w6.head_dim == 1536 and w6.kv_heads == 3 and w6.n_slots == 2
    assert sum(w6.pairs) * 2 == w6.head_dim and w6.kv_norm and w7.kv_norm
    assert abs(WL.flops_full(3600, 7200, 24, 64) / 1e9 - 159.25248) < 1e-5
    assert w7.grid == (4, 45, 80) and w7.tokens == 4 * 3600 and w7.n_slots == 2
    assert abs(WL.flops_full(14400, 28800, 24, 64) / 1e12 - 2.5480396) < 1e-6
