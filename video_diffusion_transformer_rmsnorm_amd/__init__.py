"""Python binding of libvdit (gfx950): 3D-RoPE video-DiT attention.

Argument marshalling only.  Every step runs in the HIP kernels of
``libvdit.so``; torch supplies device memory and the current stream.  The
functions carry the C ABI's names (see ``include/vdit.h``) and raise
``VditError`` on a non-OK status.  If the library has not been built the
first call raises: there is no CPU fallback.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Sequence

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG_DIR, "libvdit.so")

VDIT_OK, VDIT_ERR_INVALID_ARG, VDIT_ERR_UNSUPPORTED, VDIT_ERR_HIP = 0, 1, 2, 3
VDIT_BF16, VDIT_F32 = 0, 1
VDIT_ROPE_NO_NORM = 1
VDIT_ROPE_NO_Q_NORM = 2
VDIT_ROPE_V_NORM = 4
MODES = {"full": 0, "ring": 1, "rolling": 2, "hybrid": 3}
ABI_VERSION = 5
VDIT_ATTN_RING_FOLD = 1
VDIT_ATTN_STATE_ZERO = 2

# Every symbol include/vdit.h declares.
EXPORTS = ("vdit_rope_qk", "vdit_rope_qkv", "vdit_rms_norm", "vdit_attn_fwd", "vdit_attn_fwd_noalloc", "vdit_attn_workspace_bytes",
           "vdit_lse_merge", "vdit_last_error", "vdit_abi_version")


class VditError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"vdit status {status}: {msg}")
        self.status = status


class VditGrid(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("H", ctypes.c_int32), ("W", ctypes.c_int32),
                ("pairs_t", ctypes.c_int32), ("pairs_h", ctypes.c_int32), ("pairs_w", ctypes.c_int32),
                ("theta", ctypes.c_float)]


class VditAttnArgs(ctypes.Structure):
    _fields_ = [
        ("mode", ctypes.c_int32), ("dtype", ctypes.c_int32), ("B", ctypes.c_int32),
        ("n_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
        ("Lq", ctypes.c_int64), ("Lkv", ctypes.c_int64),
        ("scale", ctypes.c_float), ("n_kv_chunks", ctypes.c_int32),
        ("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
        ("o", ctypes.c_void_p), ("lse", ctypes.c_void_p),
        ("k_chunks", ctypes.c_void_p), ("v_chunks", ctypes.c_void_p), ("chunk_len", ctypes.c_void_p),
        ("k_cache", ctypes.c_void_p), ("v_cache", ctypes.c_void_p),
        ("frame", ctypes.c_int64), ("n_slots", ctypes.c_int32), ("flags", ctypes.c_uint32),
        ("chunk_tokens", ctypes.c_int64),
        ("state_s", ctypes.c_void_p), ("state_z", ctypes.c_void_p),
        ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t),
        ("overlap_tokens", ctypes.c_int64), ("ctx_tokens", ctypes.c_int64),
        ("key_norm_max", ctypes.c_float), ("reserved1", ctypes.c_int32),
        ("phi_coef", ctypes.c_void_p),
    ]


_lib_handle = None


def lib() -> ctypes.CDLL:
    """Load libvdit.so (once).  Raises if it is missing."""
    global _lib_handle
    if _lib_handle is None:
        _lib_handle = load(LIB_PATH)
    return _lib_handle


def load(path: str) -> ctypes.CDLL:
    """A handle on a build of the library at `path` with the ABI's signatures
    (lib() uses libvdit.so next to this file)."""
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run `python -m video_diffusion_transformer_rmsnorm_amd.build`")
    h = ctypes.CDLL(path)
    vp, i32, i64, f32, u32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_uint32
    h.vdit_rope_qk.argtypes = [vp, vp, vp, vp, i32, i64, i32, i32, i32, i32, ctypes.POINTER(VditGrid),
                               i64, i64, vp, vp, f32, u32, vp]
    h.vdit_rope_qk.restype = ctypes.c_int
    h.vdit_rope_qkv.argtypes = [vp, vp, vp, vp, vp, vp, i32, i64, i32, i32, i32, i32, ctypes.POINTER(VditGrid),
                                i64, i64, vp, vp, vp, f32, u32, vp]
    h.vdit_rope_qkv.restype = ctypes.c_int
    h.vdit_rms_norm.argtypes = [vp, vp, i32, i64, i32, i32, i32, vp, f32, vp]
    h.vdit_rms_norm.restype = ctypes.c_int
    h.vdit_attn_fwd.argtypes = [ctypes.POINTER(VditAttnArgs), vp]
    h.vdit_attn_fwd.restype = ctypes.c_int
    h.vdit_attn_fwd_noalloc.argtypes = [ctypes.POINTER(VditAttnArgs), vp]
    h.vdit_attn_fwd_noalloc.restype = ctypes.c_int
    h.vdit_attn_workspace_bytes.argtypes = [ctypes.POINTER(VditAttnArgs)]
    h.vdit_attn_workspace_bytes.restype = ctypes.c_size_t
    h.vdit_lse_merge.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i64, i32, i32, vp]
    h.vdit_lse_merge.restype = ctypes.c_int
    h.vdit_last_error.argtypes = []
    h.vdit_last_error.restype = ctypes.c_char_p
    h.vdit_abi_version.argtypes = []
    h.vdit_abi_version.restype = ctypes.c_int32
    return h


def _check(status: int):
    if status != VDIT_OK:
        raise VditError(status, lib().vdit_last_error().decode())


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return VDIT_BF16
    if t.dtype == torch.float32:
        return VDIT_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> Optional[int]:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _dev(t, name):
    if t is None:
        return
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _expect(t, name, shape, dtype=None):
    """t is None, or a tensor of exactly `shape` (and `dtype`).  The C ABI sees
    only pointers and sizes, so tensors that disagree with the sizes it is
    given would be read or written past their ends: such calls stop here."""
    if t is None:
        return
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")


def _rank(t, name, n):
    if t is not None and t.dim() != n:
        raise ValueError(f"{name} must have {n} dimensions, got shape {tuple(t.shape)}")


def make_grid(T: int, H: int, W: int, pairs: Sequence[int], theta: float = 10000.0) -> VditGrid:
    return VditGrid(T, H, W, pairs[0], pairs[1], pairs[2], theta)


def vdit_rope_qk(q, k, grid: VditGrid, q_out=None, k_out=None, token0: int = 0, t_offset: int = 0,
                 q_gain=None, k_gain=None, eps: float = 1e-6, norm: bool = True,
                 q_norm: Optional[bool] = None, stream=None):
    """Fused per-head RMSNorm + 3D-RoPE of q [B,L,Hq,D] and k [B,L,Hk,D].

    norm=False rotates only; q_norm=False (with norm=True) normalises k but
    not q, as KV-norm attention does.  Outputs default to new tensors; pass
    q_out=q / k_out=k for in-place.  Returns (q_out, k_out)."""
    import torch
    ref = q if q is not None else k
    _rank(q, "q", 4); _rank(k, "k", 4)
    B, L, _, D = ref.shape
    Hq = q.shape[2] if q is not None else 0
    Hk = k.shape[2] if k is not None else 0
    _expect(q, "q", (B, L, Hq, D), ref.dtype); _expect(q_out, "q_out", (B, L, Hq, D), ref.dtype)
    _expect(k, "k", (B, L, Hk, D), ref.dtype); _expect(k_out, "k_out", (B, L, Hk, D), ref.dtype)
    _expect(q_gain, "q_gain", (D,), torch.float32); _expect(k_gain, "k_gain", (D,), torch.float32)
    for t, n in ((q, "q"), (k, "k"), (q_out, "q_out"), (k_out, "k_out"), (q_gain, "q_gain"), (k_gain, "k_gain")):
        _dev(t, n)
    if q is not None and q_out is None:
        q_out = torch.empty_like(q)
    if k is not None and k_out is None:
        k_out = torch.empty_like(k)
    flags = 0 if norm else VDIT_ROPE_NO_NORM
    if norm and q_norm is False:
        flags |= VDIT_ROPE_NO_Q_NORM
    _check(lib().vdit_rope_qk(_ptr(q), _ptr(k), _ptr(q_out), _ptr(k_out), B, L, Hq, Hk, D,
                              _dtype_code(ref), ctypes.byref(grid), token0, t_offset,
                              _ptr(q_gain), _ptr(k_gain), eps, flags, _stream(stream)))
    return q_out, k_out


def vdit_rope_qkv(q, k, v, grid: VditGrid, q_out=None, k_out=None, v_out=None, token0: int = 0,
                  t_offset: int = 0, q_gain=None, k_gain=None, v_gain=None, eps: float = 1e-6,
                  norm: bool = True, q_norm: Optional[bool] = None, v_norm: bool = False, stream=None):
    """vdit_rope_qk of q and k plus the values v [B,L,Hk,D] in the same launch:
    v is copied to v_out, or RMS-normalised with v_gain when v_norm is set;
    never rotated.  Outputs default to new tensors.  Returns (q_out, k_out,
    v_out)."""
    import torch
    ref = q if q is not None else (k if k is not None else v)
    _rank(q, "q", 4); _rank(k, "k", 4); _rank(v, "v", 4)
    B, L, _, D = ref.shape
    Hq = q.shape[2] if q is not None else 0
    Hk = k.shape[2] if k is not None else (v.shape[2] if v is not None else 0)
    _expect(q, "q", (B, L, Hq, D), ref.dtype); _expect(q_out, "q_out", (B, L, Hq, D), ref.dtype)
    _expect(k, "k", (B, L, Hk, D), ref.dtype); _expect(k_out, "k_out", (B, L, Hk, D), ref.dtype)
    _expect(v, "v", (B, L, Hk, D), ref.dtype); _expect(v_out, "v_out", (B, L, Hk, D), ref.dtype)
    for g, n in ((q_gain, "q_gain"), (k_gain, "k_gain"), (v_gain, "v_gain")):
        _expect(g, n, (D,), torch.float32)
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (q_out, "q_out"), (k_out, "k_out"), (v_out, "v_out"),
                 (q_gain, "q_gain"), (k_gain, "k_gain"), (v_gain, "v_gain")):
        _dev(t, n)
    if q is not None and q_out is None:
        q_out = torch.empty_like(q)
    if k is not None and k_out is None:
        k_out = torch.empty_like(k)
    if v is not None and v_out is None:
        v_out = torch.empty_like(v)
    flags = 0 if norm else VDIT_ROPE_NO_NORM
    if norm and q_norm is False:
        flags |= VDIT_ROPE_NO_Q_NORM
    if v_norm:
        flags |= VDIT_ROPE_V_NORM
    _check(lib().vdit_rope_qkv(_ptr(q), _ptr(k), _ptr(v), _ptr(q_out), _ptr(k_out), _ptr(v_out), B, L, Hq, Hk, D,
                               _dtype_code(ref), ctypes.byref(grid), token0, t_offset,
                               _ptr(q_gain), _ptr(k_gain), _ptr(v_gain), eps, flags, _stream(stream)))
    return q_out, k_out, v_out


def vdit_rms_norm(x, out=None, gain=None, eps: float = 1e-6, stream=None):
    """Per-head RMSNorm of x [B,L,H,D] (the values of KV-norm attention).

    out defaults to a new tensor; out=x normalises in place.  Returns out."""
    import torch
    _rank(x, "x", 4)
    B, L, H, D = x.shape
    _expect(out, "out", x.shape, x.dtype)
    _expect(gain, "gain", (D,), torch.float32)
    for t, n in ((x, "x"), (out, "out"), (gain, "gain")):
        _dev(t, n)
    if out is None:
        out = torch.empty_like(x)
    _check(lib().vdit_rms_norm(_ptr(x), _ptr(out), B, L, H, D, _dtype_code(x), _ptr(gain), eps,
                               _stream(stream)))
    return out


def _attn_args(q, k, v, mode, o, lse, scale, n_kv_heads, Lkv) -> VditAttnArgs:
    a = VditAttnArgs()
    a.mode = MODES[mode]
    a.dtype = _dtype_code(q)
    a.B, a.Lq, a.n_heads, a.head_dim = q.shape[0], q.shape[1], q.shape[2], q.shape[3]
    a.n_kv_heads = n_kv_heads
    a.Lkv = Lkv
    a.scale = scale
    a.q, a.k, a.v, a.o, a.lse = _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse)
    return a


def vdit_attn_workspace_bytes(args: VditAttnArgs) -> int:
    n = lib().vdit_attn_workspace_bytes(ctypes.byref(args))
    if n == ctypes.c_size_t(-1).value:
        raise VditError(VDIT_ERR_INVALID_ARG, lib().vdit_last_error().decode())
    return n


def vdit_attn_fwd(q, k=None, v=None, mode: str = "full", o=None, lse=None, want_lse: bool = True,
                  scale: float = 0.0, k_chunks=None, v_chunks=None, k_cache=None, v_cache=None,
                  frame: int = 0, chunk_tokens: int = 0, state_s=None, state_z=None, workspace=None,
                  n_kv_heads: Optional[int] = None, overlap_tokens: int = 0, ctx_tokens: int = 0,
                  key_norm_max: float = 0.0, phi_coef: Optional[Sequence[float]] = None,
                  ring_fold: bool = False, state_zero: bool = False, stream=None, _noalloc: bool = False):
    """One attention call.  Returns (o, lse) (lse None unless wanted).

    full:    k, v [B,Lkv,Hk,D].
    ring:    k_chunks, v_chunks lists of [B,len_c,Hk,D]; workspace allocated if not given
             (also for full / rolling calls small enough to use the key split).
    rolling: k_cache, v_cache [B,n_slots,Lq,Hk,D]; k, v = this frame's keys/values or None
             (slot already filled); frame = stream index.
    hybrid:  k, v [B,ctx_tokens+Lq,Hk,D]; chunk_tokens; state_s [B,Hk,D,D], state_z [B,Hk,D]
             float32 (in/out); overlap_tokens keys before each chunk join its softmax
             window; the first ctx_tokens (<= overlap_tokens) keys precede the first query.
    key_norm_max: 0, or a bound on every key's norm, which replaces the library's pass
             over the keys (see vdit.h).
    phi_coef: hybrid only: 8 floats, the cubics phi_q (a0..a3) and phi_k (b0..b3) that
             replace elu + 1 in the linear term.
    ring_fold: ring only: fold the chunks one launch at a time (VDIT_ATTN_RING_FOLD).
    state_zero: hybrid only: the incoming state is zero and is not read (VDIT_ATTN_STATE_ZERO).
    """
    import torch
    if phi_coef is not None and len(phi_coef) != 8:
        raise ValueError("phi_coef: 4 coefficients of phi_q, then 4 of phi_k")
    _rank(q, "q", 4)
    B, Lq, Hq, D = q.shape
    _expect(o, "o", q.shape, q.dtype)
    _expect(lse, "lse", (B, Hq, Lq), torch.float32)
    if mode == "ring":
        if k_chunks is None or v_chunks is None or len(k_chunks) != len(v_chunks):
            raise ValueError("ring: k_chunks and v_chunks must be lists of the same length")
        for i, (kc, vc) in enumerate(zip(k_chunks, v_chunks)):
            _rank(kc, f"k_chunks[{i}]", 4)
            _expect(kc, f"k_chunks[{i}]", (B, kc.shape[1], k_chunks[0].shape[2], D), q.dtype)
            _expect(vc, f"v_chunks[{i}]", kc.shape, q.dtype)
        for i, (kc, vc) in enumerate(zip(k_chunks, v_chunks)):
            _dev(kc, f"k_chunks[{i}]"); _dev(vc, f"v_chunks[{i}]")
    elif mode == "rolling":
        _rank(k_cache, "k_cache", 5)
        if k_cache is None:
            raise ValueError("rolling: k_cache and v_cache are required")
        _expect(k_cache, "k_cache", (B, k_cache.shape[1], Lq, k_cache.shape[3], D), q.dtype)
        _expect(v_cache, "v_cache", k_cache.shape, q.dtype)
        _expect(k, "k", (B, Lq, k_cache.shape[3], D), q.dtype)
        _expect(v, "v", (B, Lq, k_cache.shape[3], D), q.dtype)
    elif k is not None:
        _rank(k, "k", 4)
        _expect(k, "k", (B, k.shape[1], k.shape[2], D), q.dtype)
        _expect(v, "v", k.shape, q.dtype)
        if mode == "hybrid":
            Hk = k.shape[2]
            _expect(state_s, "state_s", (B, Hk, D, D), torch.float32)
            _expect(state_z, "state_z", (B, Hk, D), torch.float32)
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (o, "o"), (lse, "lse"), (k_cache, "k_cache"),
                 (v_cache, "v_cache"), (state_s, "state_s"), (state_z, "state_z"), (workspace, "workspace")):
        _dev(t, n)
    if o is None:
        o = torch.empty_like(q)
    if lse is None and want_lse:
        lse = torch.empty((B, Hq, Lq), dtype=torch.float32, device=q.device)
    keep = []
    if mode == "ring":
        hk = k_chunks[0].shape[2]
        lens = [int(c.shape[1]) for c in k_chunks]
        a = _attn_args(q, None, None, mode, o, lse, scale, n_kv_heads or hk, sum(lens))
        n = len(k_chunks)
        kp = (ctypes.c_void_p * n)(*[c.data_ptr() for c in k_chunks])
        vp = (ctypes.c_void_p * n)(*[c.data_ptr() for c in v_chunks])
        ln = (ctypes.c_int64 * n)(*lens)
        keep += [kp, vp, ln]
        a.n_kv_chunks = n
        a.k_chunks = ctypes.cast(kp, ctypes.c_void_p)
        a.v_chunks = ctypes.cast(vp, ctypes.c_void_p)
        a.chunk_len = ctypes.cast(ln, ctypes.c_void_p)
    elif mode == "rolling":
        hk = k_cache.shape[3]
        a = _attn_args(q, k, v, mode, o, lse, scale, n_kv_heads or hk, 0)
        a.k_cache, a.v_cache = _ptr(k_cache), _ptr(v_cache)
        a.n_slots = k_cache.shape[1]
        a.frame = frame
    elif mode == "hybrid":
        hk = k.shape[2]
        a = _attn_args(q, k, v, mode, o, lse, scale, n_kv_heads or hk, k.shape[1])
        a.chunk_tokens = chunk_tokens
        a.state_s, a.state_z = _ptr(state_s), _ptr(state_z)
        a.overlap_tokens, a.ctx_tokens = overlap_tokens, ctx_tokens
    else:
        hk = k.shape[2]
        a = _attn_args(q, k, v, mode, o, lse, scale, n_kv_heads or hk, k.shape[1])
    a.key_norm_max = key_norm_max
    if ring_fold:
        a.flags |= VDIT_ATTN_RING_FOLD
    if state_zero:
        a.flags |= VDIT_ATTN_STATE_ZERO
    if phi_coef is not None:
        coef = (ctypes.c_float * 8)(*[float(c) for c in phi_coef])
        keep.append(coef)
        a.phi_coef = ctypes.cast(coef, ctypes.c_void_p)
    if _noalloc:
        _check(lib().vdit_attn_fwd_noalloc(ctypes.byref(a), _stream(stream)))
        del keep
        return o, lse
    need = vdit_attn_workspace_bytes(a)
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    if workspace is not None:
        a.workspace = workspace.data_ptr()
        a.workspace_bytes = workspace.numel() * workspace.element_size()
    _check(lib().vdit_attn_fwd(ctypes.byref(a), _stream(stream)))
    del keep
    return o, lse


def vdit_attn_fwd_noalloc(q, k=None, v=None, mode: str = "full", o=None, lse=None, **kw):
    """vdit_attn_fwd with the library's own device scratch as the workspace
    (no workspace argument, nothing allocated by the library; o and lse must
    be passed, or are allocated here by torch).  Same arguments otherwise."""
    if kw.get("workspace") is not None:
        raise ValueError("vdit_attn_fwd_noalloc takes no workspace")
    return vdit_attn_fwd(q, k, v, mode=mode, o=o, lse=lse, _noalloc=True, **kw)


def vdit_lse_merge(o_a, lse_a, o_b, lse_b, o_out=None, lse_out=None, out_dtype=None, stream=None):
    """Merge two attention partials; returns (o_out, lse_out)."""
    import torch
    _rank(o_a, "o_a", 4)
    B, L, H, D = o_a.shape
    _expect(o_b, "o_b", o_a.shape, o_a.dtype)
    for t, n in ((lse_a, "lse_a"), (lse_b, "lse_b"), (lse_out, "lse_out")):
        _expect(t, n, (B, H, L), torch.float32)
    _expect(o_out, "o_out", o_a.shape)
    for t, n in ((o_a, "o_a"), (lse_a, "lse_a"), (o_b, "o_b"), (lse_b, "lse_b"), (o_out, "o_out"), (lse_out, "lse_out")):
        _dev(t, n)
    if o_out is None:
        o_out = torch.empty(o_a.shape, dtype=out_dtype or o_a.dtype, device=o_a.device)
    if lse_out is None:
        lse_out = torch.empty_like(lse_a)
    _check(lib().vdit_lse_merge(_ptr(o_a), _ptr(lse_a), _ptr(o_b), _ptr(lse_b), _ptr(o_out), _ptr(lse_out),
                                _dtype_code(o_a), _dtype_code(o_out), B, L, H, D, _stream(stream)))
    return o_out, lse_out


def default_scale(D: int) -> float:
    return 1.0 / math.sqrt(D)


__all__ = ["VDIT_ATTN_RING_FOLD", "VDIT_ATTN_STATE_ZERO", "VDIT_ROPE_V_NORM", "vdit_rope_qk", "vdit_rope_qkv", "vdit_rms_norm", "vdit_attn_fwd", "vdit_attn_fwd_noalloc", "vdit_lse_merge", "vdit_attn_workspace_bytes", "make_grid",
           "VditGrid", "VditAttnArgs", "VditError", "lib", "EXPORTS", "LIB_PATH"]
