"""Plain float64 CPU oracle for 3D-RoPE video-DiT attention.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this module.  The HIP library never calls it and
shares no code with it: this file uses numpy only and writes every step as
its plain mathematical definition, in float64, with no tiling, online softmax
or fusion.

How it is pinned (tests/test_oracle_pins.py): every function is checked
against something other than itself -- closed forms, invariances the pages
state, brute-force loops on tiny inputs, hand-derived rotations and torch
float64 attention.  Against the pages themselves parity is unpinned: no page
prints a worked numerical example to compare with.

Layouts follow the library: q, k, v, o are ``[B, L, H, D]`` row-major;
log-sum-exp values are ``[B, H, L]``; linear-attention state is ``s [B, Hk, D, D]``
(index order: feature of phi(k), value channel) and ``z [B, Hk, D]``.

Sources (pages by title, with the passage each step follows):
  * FlashDecoder: Real-Time Latent-to-Pixel Streaming Decoder with
    Transformers -- Sec. 3.2 "Base Architecture" (RMSNorm, GQA, 3D-RoPE applied
    separately to the temporal and spatial axes), Sec. 3.3 (rolling KV cache,
    the sliding-window attention pattern, processing order instead of masks),
    Sec. 3.4 "Step 2: Temporal Refinement" (the same streaming with r_t
    sub-frames per step and a window of r_t * W_frm sub-frames),
    Sec. 4 "Long Video Decoding" (RoPE positions relative to the window).
    It cites RoFormer for rotary embeddings and Zhang & Sennrich for RMSNorm;
    the rotation and the norm below are those papers' definitions.
  * ReGenVC: End-to-End Real-Time Generative Video Coding at Ultra-Low
    Bitrate -- unified sequence parallelism paragraph (Sec. 3.5 by the page's
    cross references): ring attention combines key/value blocks in an
    online-softmax fashion and is exact up to reduction order.
  * MobileWan: Closing the Quality Gap for Mobile Video Diffusion (Pith
    review) -- hybrid attention: softmax inside a chunk, causal linear
    attention across chunks with running state (s_t, z_t); the recurrent
    form is the standard equivalence of causal linear attention (review of
    Sec. 3.2, Eq. 3 and Eqs. 5-10; the equations themselves are not printed).

Readings taken where the pages are silent (each is also listed in the design
notes): adjacent channel pairs; axis blocks in the order t, h, w; per-axis
frequency theta^(-j/P_a); tokens flattened t-major then h then w; RMSNorm per
head with eps=1e-6 and unit gain by default; softmax scale 1/sqrt(D) by
default; natural-log LSE with -inf for an empty key set; phi = elu + 1 applied
to the post-norm, post-rotation q and k without the softmax scale; the
hybrid's stabiliser c_t cancels (joint normalisation of both terms); KV-norm
is a per-head RMSNorm of keys and values with queries left un-normalised; a
temporal-refinement step holds the r_t sub-frames of one latent frame, which
take consecutive window-relative temporal positions.
"""
from __future__ import annotations

import math
from typing import Optional, Sequence, Tuple

import numpy as np

_QBLOCK = 1024  # query rows per materialised score block (memory bound only)


# ------------------------------------------------------------ positions --

def grid_positions(n_tokens: int, grid: Tuple[int, int, int], token0: int = 0,
                   t_offset: int = 0) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Grid coordinates (t, h, w) of tokens token0 .. token0+n_tokens-1.

    Tokens of a T x H x W latent grid are flattened t-major, then h, then w
    (FlashDecoder Sec. 3.1 writes latents as T' x H' x W'; the flattening
    order itself is a reading).  ``t_offset`` is added to every t.
    """
    T, H, W = grid
    n = token0 + np.arange(n_tokens, dtype=np.int64)
    t = n // (H * W) + t_offset
    h = (n // W) % H
    w = n % W
    return t, h, w


# --------------------------------------------------------------- RMSNorm --

def rmsnorm(x: np.ndarray, eps: float = 1e-6, gain: Optional[np.ndarray] = None) -> np.ndarray:
    """RMSNorm over the last axis: x / sqrt(mean(x^2) + eps) * g.

    Zhang & Sennrich's root-mean-square layer normalisation, cited by
    FlashDecoder Sec. 3.2 "Base Architecture"; applied per (token, head).
    """
    x = np.asarray(x, dtype=np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    y = x / np.sqrt(ms + eps)
    if gain is not None:
        y = y * np.asarray(gain, dtype=np.float64)
    return y


# ------------------------------------------------------------------ RoPE --

def rope_frequencies(pairs: Sequence[int], theta: float = 10000.0):
    """Per channel pair: (axis id 0/1/2 for t/h/w, angular frequency omega).

    The D/2 channel pairs are split, in order, into blocks of P_t, P_h, P_w
    pairs; each block is an independent 1D rotary embedding of dimension
    2*P_a along its own axis (FlashDecoder Sec. 3.2: 3D-RoPE applied
    separately to the temporal and spatial dimensions), with RoFormer's
    frequencies theta^(-2j / (2 P_a)) = theta^(-j / P_a), j = 0 .. P_a - 1.
    """
    axis = []
    omega = []
    for a, Pa in enumerate(pairs):
        for j in range(Pa):
            axis.append(a)
            omega.append(theta ** (-j / Pa))
    return np.asarray(axis, dtype=np.int64), np.asarray(omega, dtype=np.float64)


def rope_angles(t: np.ndarray, h: np.ndarray, w: np.ndarray, pairs: Sequence[int],
                theta: float = 10000.0) -> np.ndarray:
    """Rotation angle alpha[token, pair] = position along the pair's axis * omega."""
    axis, omega = rope_frequencies(pairs, theta)
    pos = np.stack([np.asarray(t, np.float64), np.asarray(h, np.float64),
                    np.asarray(w, np.float64)], axis=1)          # [L, 3]
    return pos[:, axis] * omega[None, :]                          # [L, P]


def rope_rotate(x: np.ndarray, alpha: np.ndarray) -> np.ndarray:
    """Rotate adjacent channel pairs (x_2p, x_2p+1) by alpha[token, p].

    x is [B, L, H, D]; alpha is [L, D/2].  (x0, x1) -> (x0 cos a - x1 sin a,
    x0 sin a + x1 cos a), i.e. multiplication of x0 + i x1 by e^{i a}
    (RoFormer's rotary embedding, cited by FlashDecoder Sec. 3.2).
    """
    x = np.asarray(x, dtype=np.float64)
    c = np.cos(alpha)[None, :, None, :]
    s = np.sin(alpha)[None, :, None, :]
    x0 = x[..., 0::2]
    x1 = x[..., 1::2]
    y = np.empty_like(x)
    y[..., 0::2] = x0 * c - x1 * s
    y[..., 1::2] = x0 * s + x1 * c
    return y


def rope_qk(q: np.ndarray, k: np.ndarray, grid, pairs, theta: float = 10000.0,
            token0: int = 0, t_offset: int = 0, eps: float = 1e-6, norm: bool = True,
            q_gain=None, k_gain=None, q_norm: Optional[bool] = None):
    """Per-head RMSNorm of q and k (not v), then 3D-RoPE at each token's grid position.

    q_norm=False leaves q un-normalised while k still is: the query side of
    FlashDecoder's KV-norm (Sec. 3.2 "Base Architecture" normalises keys and
    values inside attention, not queries).  q_norm=None follows `norm`.
    """
    L = q.shape[1]
    t, h, w = grid_positions(L, grid, token0, t_offset)
    alpha = rope_angles(t, h, w, pairs, theta)
    q_norm = norm if q_norm is None else q_norm
    qn = rmsnorm(q, eps, q_gain) if q_norm else np.asarray(q, np.float64)
    kn = rmsnorm(k, eps, k_gain) if norm else np.asarray(k, np.float64)
    return rope_rotate(qn, alpha), rope_rotate(kn, alpha)


# ------------------------------------------------------------- attention --

def _kv_head(h: int, Hq: int, Hk: int) -> int:
    """GQA: query head h reads key/value head h // (Hq / Hk) (FlashDecoder Sec. 3.2)."""
    return h // (Hq // Hk)


def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: Optional[float] = None):
    """Exact softmax attention, no mask.

    O[i] = sum_j softmax_j(scale * q_i . k_j) v_j and
    LSE[i] = ln sum_j exp(scale * q_i . k_j) (natural log).  An empty key set
    gives O = 0 and LSE = -inf.  Returns (o [B,Lq,Hq,D], lse [B,Hq,Lq]).
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    B, Lq, Hq, D = q.shape
    Lk, Hk = k.shape[1], k.shape[2]
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    o = np.zeros((B, Lq, Hq, D))
    lse = np.full((B, Hq, Lq), -np.inf)
    if Lk == 0:
        return o, lse
    for b in range(B):
        for h in range(Hq):
            kh = _kv_head(h, Hq, Hk)
            K = k[b, :, kh, :]
            V = v[b, :, kh, :]
            for r0 in range(0, Lq, _QBLOCK):
                Q = q[b, r0:r0 + _QBLOCK, h, :]
                s = scale * (Q @ K.T)
                m = s.max(axis=1, keepdims=True)
                e = np.exp(s - m)
                l = e.sum(axis=1, keepdims=True)
                o[b, r0:r0 + _QBLOCK, h, :] = (e @ V) / l
                lse[b, h, r0:r0 + _QBLOCK] = (m + np.log(l))[:, 0]
    return o, lse


def attention_probs(q: np.ndarray, k: np.ndarray, scale: Optional[float] = None) -> np.ndarray:
    """Softmax weight matrix P[b, h, i, j] (small inputs only)."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    B, Lq, Hq, D = q.shape
    Hk = k.shape[2]
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    P = np.zeros((B, Hq, Lq, k.shape[1]))
    for b in range(B):
        for h in range(Hq):
            s = scale * (q[b, :, h, :] @ k[b, :, _kv_head(h, Hq, Hk), :].T)
            e = np.exp(s - s.max(axis=1, keepdims=True))
            P[b, h] = e / e.sum(axis=1, keepdims=True)
    return P


# ------------------------------------------------------------- LSE merge --

def lse_merge(o_a, lse_a, o_b, lse_b):
    """Combine two attention partials over disjoint key sets.

    L = ln(e^{L_a} + e^{L_b}); O = e^{L_a - L} O_a + e^{L_b - L} O_b.  A partial
    with L = -inf has weight 0; two empty partials give O = 0, L = -inf.
    This is the online-softmax combination ring attention uses (ReGenVC,
    USP paragraph).  o: [B, L, H, D]; lse: [B, H, L].
    """
    o_a = np.asarray(o_a, np.float64)
    o_b = np.asarray(o_b, np.float64)
    la = np.asarray(lse_a, np.float64)
    lb = np.asarray(lse_b, np.float64)
    L = np.logaddexp(la, lb)
    with np.errstate(invalid="ignore"):
        wa = np.where(np.isneginf(la), 0.0, np.exp(la - L))
        wb = np.where(np.isneginf(lb), 0.0, np.exp(lb - L))
    wa = np.nan_to_num(wa)
    wb = np.nan_to_num(wb)
    # weights [B,H,L] -> [B,L,H,1]
    wa_t = np.transpose(wa, (0, 2, 1))[..., None]
    wb_t = np.transpose(wb, (0, 2, 1))[..., None]
    return wa_t * o_a + wb_t * o_b, L


# ------------------------------------------------------------------ ring --

def ring_attention(q, k_chunks, v_chunks, scale: Optional[float] = None):
    """Ring attention replayed on one device: attend to each key/value chunk in
    turn and fold the partials with ``lse_merge`` left to right (ReGenVC, USP
    paragraph: key/value blocks combined in an online-softmax fashion)."""
    o, lse = attention(q, k_chunks[0], v_chunks[0], scale)
    for kc, vc in zip(k_chunks[1:], v_chunks[1:]):
        oc, lc = attention(q, kc, vc, scale)
        o, lse = lse_merge(o, lse, oc, lc)
    return o, lse


# --------------------------------------------------------------- rolling --

def rolling_window(f: int, n_slots: int) -> range:
    """Frames a query frame f attends to: the most recent n_slots frames,
    f0 = max(0, f - n_slots + 1) .. f (FlashDecoder Sec. 3.3, "Attention
    Pattern"; warm-up frames see fewer frames, without padding)."""
    return range(max(0, f - n_slots + 1), f + 1)


def rolling_frame(q_frames, k_frames, v_frames, f: int, n_slots: int, frame_grid,
                  pairs, theta: float = 10000.0, eps: float = 1e-6, norm: bool = True,
                  scale: Optional[float] = None, kv_norm: bool = False):
    """Output of step f of a step-by-step stream with a rolling KV window.

    Inputs are the raw (pre-norm, pre-rotation) per-step tensors
    [F, L_step, H, D]; a step covers the grid frame_grid = (T_step, H, W),
    T_step temporal positions of H x W tokens each.  T_step = 1 is
    FlashDecoder's frame-by-frame decode (Sec. 3.3); T_step = r_t is its
    temporal refinement (Sec. 3.4, Step 2), where one step carries the r_t
    upsampled sub-frames of a latent frame and the window of n_slots steps
    spans r_t * n_slots sub-frames.  Every step u in the window is normalised
    and rotated with temporal positions relative to the window start,
    t = T_step * (u - f0) + s for its sub-frame s (FlashDecoder Sec. 4
    "Long Video Decoding"), and (h, w) from the step's own grid.  q_f
    attends to the concatenated window with no mask.

    kv_norm=True is FlashDecoder's KV-norm (Sec. 3.2): per-head RMSNorm of
    keys (before rotation) and values; queries are rotated only.  Otherwise
    q and k are normalised when `norm` is set and v is left as is.
    Returns (o [1, L_step, H, D], lse [1, H, L_step]).
    """
    win = list(rolling_window(f, n_slots))
    f0 = win[0]
    t_step = int(frame_grid[0])
    ks, vs = [], []
    qf = None
    for u in win:
        qu, ku = rope_qk(q_frames[u][None], k_frames[u][None], frame_grid, pairs, theta,
                         token0=0, t_offset=t_step * (u - f0), eps=eps, norm=norm or kv_norm,
                         q_norm=False if kv_norm else None)
        ks.append(ku)
        vu = np.asarray(v_frames[u][None], np.float64)
        vs.append(rmsnorm(vu, eps) if kv_norm else vu)
        if u == f:
            qf = qu
    K = np.concatenate(ks, axis=1)
    V = np.concatenate(vs, axis=1)
    return attention(qf, K, V, scale)


# ---------------------------------------------------------------- hybrid --

def phi(x: np.ndarray) -> np.ndarray:
    """Feature map elu(x) + 1: x + 1 for x > 0, e^x otherwise (strictly positive)."""
    x = np.asarray(x, np.float64)
    return np.where(x > 0, x + 1.0, np.exp(np.minimum(x, 0.0)))


def phi_poly(x: np.ndarray, coef: Sequence[float]) -> np.ndarray:
    """Degree-3 polynomial feature map c0 + c1 x + c2 x^2 + c3 x^3, element-wise.

    The MobileWan review's ledger gives the linear attention's feature maps
    phi_q and phi_k as learnable polynomials of degree 3 (Appendix A.3.1 as
    the ledger quotes it) and no coefficients; here they are inputs.  For the
    normaliser phi_q(q)^T z to stay positive the coefficients must keep the
    polynomial positive on the values it is fed.
    """
    x = np.asarray(x, np.float64)
    c = [float(a) for a in coef]
    return c[0] + c[1] * x + c[2] * x ** 2 + c[3] * x ** 3


def _feature_maps(phi_coef):
    """(phi_q, phi_k): elu + 1 for both when phi_coef is None, else the two
    cubics of phi_coef = (a0, a1, a2, a3, b0, b1, b2, b3)."""
    if phi_coef is None:
        return phi, phi
    c = [float(a) for a in phi_coef]
    if len(c) != 8:
        raise ValueError("phi_coef holds 4 coefficients for phi_q, then 4 for phi_k")
    return (lambda x: phi_poly(x, c[:4])), (lambda x: phi_poly(x, c[4:]))


def _chunks(L: int, chunk_tokens: int):
    return [(c0, min(c0 + chunk_tokens, L)) for c0 in range(0, L, chunk_tokens)]


def _merge_softmax_linear(o_s, lse_s, num_lin, den_lin):
    """Joint normalisation of a softmax partial and a linear-attention partial.

    (sum_j e^{s_ij} v_j + phi(q_i)^T S) / (sum_j e^{s_ij} + phi(q_i)^T z), written
    as an LSE merge with L_lin = ln(phi(q)^T z) and O_lin = phi(q)^T S / phi(q)^T z.
    o_s [n, D]; lse_s [n]; num_lin [n, D]; den_lin [n].
    """
    with np.errstate(divide="ignore", invalid="ignore"):
        lse_l = np.where(den_lin > 0, np.log(np.where(den_lin > 0, den_lin, 1.0)), -np.inf)
        o_l = np.where(den_lin[:, None] > 0, num_lin / np.where(den_lin > 0, den_lin, 1.0)[:, None], 0.0)
    L = np.logaddexp(lse_s, lse_l)
    wa = np.where(np.isneginf(lse_s), 0.0, np.exp(lse_s - L))
    wb = np.where(np.isneginf(lse_l), 0.0, np.exp(lse_l - L))
    return wa[:, None] * o_s + wb[:, None] * o_l, L


def _window(c0: int, c1: int, ctx: int, overlap: int):
    """Keys a query chunk [c0, c1) (query indices) attends to with softmax: its
    own tokens plus the `overlap` tokens before them, in key indices of a call
    whose first `ctx` keys precede the first query (MobileWan review, Appendix
    A.3.1 as the ledger quotes it: chunk T_c, overlap T_o temporal slices for
    the softmax attention)."""
    return max(0, ctx + c0 - overlap), ctx + c1


def _folded_end(Lkv: int, overlap: int) -> int:
    """Keys the returned state covers: all but the last `overlap`, which the
    next call passes back as its context."""
    return max(0, Lkv - overlap)


def _hybrid_args(q, k, v, scale, s0, z0, ctx, overlap):
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    B, L, Hq, D = q.shape
    Hk = k.shape[2]
    if k.shape[1] != ctx + L or v.shape[1] != ctx + L:
        raise ValueError("k and v hold ctx + Lq tokens")
    if not 0 <= ctx <= overlap:
        raise ValueError("0 <= ctx <= overlap")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    s0 = np.zeros((B, Hk, D, D)) if s0 is None else np.array(s0, np.float64)
    z0 = np.zeros((B, Hk, D)) if z0 is None else np.array(z0, np.float64)
    return q, k, v, scale, s0, z0


def hybrid_explicit(q, k, v, chunk_tokens: int, scale: Optional[float] = None,
                    s0=None, z0=None, overlap: int = 0, ctx: int = 0, phi_coef=None):
    """Chunk-hybrid attention, explicit form (MobileWan review, Sec. 3.2).

    Query token i in chunk c = [c*C, (c+1)*C) attends with softmax to the keys
    of its window W_c (its own chunk, bidirectional, plus the `overlap`
    tokens before it; Appendix A.3.1's T_o) and, through linear attention
    with phi = elu + 1, to every key before that window:
        O_i = (sum_{j in W_c} e^{s_ij} v_j + sum_{j < start(W_c)} (phi(q_i).phi(k_j)) v_j)
              / (sum_{j in W_c} e^{s_ij} + sum_{j < start(W_c)} phi(q_i).phi(k_j)),
    with s_ij = scale q_i.k_j, so each earlier key enters once.  k and v hold
    ctx + Lq tokens: the first ctx (at most `overlap`) are context from before
    the first query.  The incoming state (s0, z0) stands for keys before this
    call; the earlier-key sums are formed directly from all earlier keys (no
    running state).  The returned state adds every key but the last
    `overlap`.  phi_coef (8 floats) replaces elu + 1 by the degree-3
    polynomials phi_q, phi_k (see phi_poly).  Returns (o, lse, s_final, z_final).
    """
    q, k, v, scale, s0, z0 = _hybrid_args(q, k, v, scale, s0, z0, ctx, overlap)
    B, L, Hq, D = q.shape
    Hk = k.shape[2]
    o = np.zeros((B, L, Hq, D))
    lse = np.zeros((B, Hq, L))
    phi_q, phi_k = _feature_maps(phi_coef)
    fq = phi_q(q)
    fk = phi_k(k)
    for b in range(B):
        for h in range(Hq):
            kh = _kv_head(h, Hq, Hk)
            for c0, c1 in _chunks(L, chunk_tokens):
                w0, w1 = _window(c0, c1, ctx, overlap)
                os_, ls_ = attention(q[b:b + 1, c0:c1, h:h + 1], k[b:b + 1, w0:w1, kh:kh + 1],
                                     v[b:b + 1, w0:w1, kh:kh + 1], scale)
                S = s0[b, kh] + fk[b, :w0, kh, :].T @ v[b, :w0, kh, :]
                z = z0[b, kh] + fk[b, :w0, kh, :].sum(axis=0)
                num = fq[b, c0:c1, h, :] @ S
                den = fq[b, c0:c1, h, :] @ z
                oc, lc = _merge_softmax_linear(os_[0, :, 0, :], ls_[0, 0, :], num, den)
                o[b, c0:c1, h, :] = oc
                lse[b, h, c0:c1] = lc
    e = _folded_end(k.shape[1], overlap)
    s_fin = s0 + np.einsum("blhd,blhe->bhde", fk[:, :e], v[:, :e])
    z_fin = z0 + fk[:, :e].sum(axis=1)
    return o, lse, s_fin, z_fin


def hybrid_recurrent(q, k, v, chunk_tokens: int, scale: Optional[float] = None,
                     s0=None, z0=None, overlap: int = 0, ctx: int = 0, phi_coef=None):
    """Chunk-hybrid attention run as an RNN over chunks (MobileWan review,
    Sec. 3.2, Eqs. 5-10 as described): for each chunk, first absorb into the
    running state (s_t, z_t) the keys that now fall before the chunk's
    softmax window (s += phi(k_j) v_j^T, z += phi(k_j)), then read it for the
    cross-chunk term; at the end absorb all keys but the last `overlap`.
    Window, context, overlap and phi_coef as in hybrid_explicit.  Returns (o, lse, s, z)."""
    q, k, v, scale, s, z = _hybrid_args(q, k, v, scale, s0, z0, ctx, overlap)
    B, L, Hq, D = q.shape
    Hk = k.shape[2]
    o = np.zeros((B, L, Hq, D))
    lse = np.zeros((B, Hq, L))
    phi_q, phi_k = _feature_maps(phi_coef)
    pos = 0  # keys absorbed so far

    def absorb(upto):
        nonlocal s, z, pos
        if upto > pos:
            fk = phi_k(k[:, pos:upto])
            s = s + np.einsum("blhd,blhe->bhde", fk, v[:, pos:upto])
            z = z + fk.sum(axis=1)
            pos = upto

    for c0, c1 in _chunks(L, chunk_tokens):
        w0, w1 = _window(c0, c1, ctx, overlap)
        absorb(w0)
        os_, ls_ = attention(q[:, c0:c1], k[:, w0:w1], v[:, w0:w1], scale)
        fq = phi_q(q[:, c0:c1])
        for b in range(B):
            for h in range(Hq):
                kh = _kv_head(h, Hq, Hk)
                num = fq[b, :, h, :] @ s[b, kh]
                den = fq[b, :, h, :] @ z[b, kh]
                oc, lc = _merge_softmax_linear(os_[b, :, h, :], ls_[b, h, :], num, den)
                o[b, c0:c1, h, :] = oc
                lse[b, h, c0:c1] = lc
    absorb(_folded_end(k.shape[1], overlap))
    return o, lse, s, z


def hybrid_partials(q, k, v, chunk_tokens: int, scale: Optional[float] = None, s0=None, z0=None,
                    overlap: int = 0, ctx: int = 0, phi_coef=None):
    """The two partials of the hybrid, per token: softmax (o_s, lse_s) over the
    token's window and linear (o_l, lse_l) over the keys before it, with
    lse_l = ln(phi_q(q)^T z) (-inf when that is not positive, e.g. z = 0).
    Used to check each partial on its own."""
    q, k, v, scale, s0, z0 = _hybrid_args(q, k, v, scale, s0, z0, ctx, overlap)
    B, L, Hq, D = q.shape
    Hk = k.shape[2]
    o_s = np.zeros((B, L, Hq, D)); l_s = np.zeros((B, Hq, L))
    o_l = np.zeros((B, L, Hq, D)); l_l = np.full((B, Hq, L), -np.inf)
    phi_q, phi_k = _feature_maps(phi_coef)
    fq = phi_q(q); fk = phi_k(k)
    for c0, c1 in _chunks(L, chunk_tokens):
        w0, w1 = _window(c0, c1, ctx, overlap)
        oc, lc = attention(q[:, c0:c1], k[:, w0:w1], v[:, w0:w1], scale)
        o_s[:, c0:c1] = oc
        l_s[:, :, c0:c1] = lc
        for b in range(B):
            for h in range(Hq):
                kh = _kv_head(h, Hq, Hk)
                S = s0[b, kh] + fk[b, :w0, kh, :].T @ v[b, :w0, kh, :]
                z = z0[b, kh] + fk[b, :w0, kh, :].sum(axis=0)
                den = fq[b, c0:c1, h, :] @ z
                num = fq[b, c0:c1, h, :] @ S
                pos = den > 0
                o_l[b, c0:c1, h, :][pos] = num[pos] / den[pos][:, None]
                l_l[b, h, c0:c1][pos] = np.log(den[pos])
    return o_s, l_s, o_l, l_l


__all__ = [
    "grid_positions", "rmsnorm", "rope_frequencies", "rope_angles", "rope_rotate", "rope_qk",
    "attention", "attention_probs", "lse_merge", "ring_attention", "rolling_window",
    "rolling_frame", "phi", "phi_poly", "hybrid_explicit", "hybrid_recurrent", "hybrid_partials",
]
