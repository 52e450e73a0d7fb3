"""CPU-only checks of the C-ABI library: it loads, exports every declared
symbol, its structs match the Python mirror, and argument validation rejects
bad calls before touching the GPU.  No compute call is made here."""
import ctypes
import os
import re
import shutil
import subprocess

import pytest

import video_diffusion_transformer_rmsnorm_amd as V
import workloads as WL

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "vdit.h")
CSRC = os.path.join(ROOT, "video_diffusion_transformer_rmsnorm_amd", "csrc")
HOST = os.path.join(ROOT, "tests", "host")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(vdit_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(V.LIB_PATH):
        pytest.fail("libvdit.so is not built (run __graft_entry__.build())")
    return V.lib()


def test_header_declares_the_binding_exports():
    assert _declared_functions() == sorted(V.EXPORTS)


def test_library_exports_every_declared_symbol(lib):
    for name in _declared_functions():
        assert hasattr(lib, name), name
    nm = shutil.which("nm")
    if nm:
        out = subprocess.run([nm, "-D", "--defined-only", V.LIB_PATH], capture_output=True, text=True).stdout
        syms = {line.split()[-1] for line in out.splitlines() if line.strip()}
        for name in _declared_functions():
            assert name in syms, name


def test_abi_version(lib):
    assert lib.vdit_abi_version() == V.ABI_VERSION == 5


def test_struct_layout_matches_header(tmp_path):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    exe = tmp_path / "layout"
    cmd = [gcc, "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"), "-I", "/opt/rocm/include",
           os.path.join(HOST, "layout_probe.c"), "-o", str(exe)]
    subprocess.run(cmd, check=True, capture_output=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout
    vals = dict(line.split() for line in out.splitlines())
    assert int(vals["vdit_grid"]) == ctypes.sizeof(V.VditGrid)
    assert int(vals["vdit_attn_args"]) == ctypes.sizeof(V.VditAttnArgs)
    for name, _ in V.VditAttnArgs._fields_:
        assert int(vals[name]) == getattr(V.VditAttnArgs, name).offset, name


def test_host_validation_under_sanitizers(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not available")
    exe = tmp_path / "validate_test"
    base = [gxx, "-std=c++17", "-O1", "-g", "-I", CSRC, os.path.join(HOST, "validate_test.cpp"), "-o", str(exe)]
    san = base[:1] + ["-fsanitize=address,undefined", "-fno-omit-frame-pointer"] + base[1:]
    r = subprocess.run(san, capture_output=True, text=True)
    if r.returncode != 0:  # sanitizer runtime missing: plain build
        subprocess.run(base, check=True, capture_output=True)
    run = subprocess.run([str(exe)], capture_output=True, text=True,
                         env={**os.environ, "ASAN_OPTIONS": "detect_leaks=0"})
    assert run.returncode == 0, run.stdout + run.stderr
    assert "validate_test ok" in run.stdout


def _status(lib, fn, *args):
    st = fn(*args)
    return st, lib.vdit_last_error().decode()


def test_rope_validation_errors_return_before_any_gpu_call(lib):
    grid = V.make_grid(21, 30, 52, (22, 21, 21))
    fake = 1 << 20  # never dereferenced: validation fails first
    st, msg = _status(lib, lib.vdit_rope_qk, fake, None, fake, None, 1, 100, 12, 12, 96, 0,
                      ctypes.byref(grid), 0, 0, None, None, 1e-6, 0, None)
    assert st == V.VDIT_ERR_UNSUPPORTED and "head_dim" in msg
    bad = V.make_grid(21, 30, 52, (22, 21, 20))
    st, msg = _status(lib, lib.vdit_rope_qk, fake, None, fake, None, 1, 100, 12, 12, 128, 0,
                      ctypes.byref(bad), 0, 0, None, None, 1e-6, 0, None)
    assert st == V.VDIT_ERR_INVALID_ARG and "pairs" in msg
    st, msg = _status(lib, lib.vdit_rope_qk, fake + 2, None, fake + 2, None, 1, 100, 12, 12, 128, 0,
                      ctypes.byref(grid), 0, 0, None, None, 1e-6, 0, None)
    assert st == V.VDIT_ERR_INVALID_ARG and "aligned" in msg
    st, msg = _status(lib, lib.vdit_rope_qk, fake, None, fake, None, 1, 100, 12, 12, 128, 0,
                      ctypes.byref(grid), 0, 0, None, None, 1e-6, 8, None)
    assert st == V.VDIT_ERR_INVALID_ARG and "flags" in msg


def test_rope_qkv_validation_errors_return_before_any_gpu_call(lib):
    grid = V.make_grid(21, 30, 52, (22, 21, 21))
    a, b, c = 1 << 24, 1 << 26, 1 << 28  # never dereferenced: validation fails first
    nk = 100 * 12 * 128 * 2  # bytes of one [1, 100, 12, 128] bf16 tensor

    def qkv(q_in, k_in, v_in, q_out, k_out, v_out, Hq=12, Hk=12, v_gain=None, flags=0):
        return _status(lib, lib.vdit_rope_qkv, q_in, k_in, v_in, q_out, k_out, v_out, 1, 100, Hq, Hk, 128, 0,
                       ctypes.byref(grid), 0, 0, None, None, v_gain, 1e-6, flags, None)
    st, msg = qkv(a, b, c, a, b, None)
    assert st == V.VDIT_ERR_INVALID_ARG and "v_in and v_out" in msg
    st, msg = qkv(a, b, c, a, b, b + nk - 64)  # the values' output runs into the keys' output
    assert st == V.VDIT_ERR_INVALID_ARG and "v_out overlaps" in msg
    st, msg = qkv(a, b, c, a, b, a + 1024)  # ... into the queries
    assert st == V.VDIT_ERR_INVALID_ARG and "v_out overlaps" in msg
    st, msg = qkv(a, b, c, c + 4096, b, 1 << 30)  # the queries' output over the values' input
    assert st == V.VDIT_ERR_INVALID_ARG and "overlaps v_in" in msg
    st, msg = qkv(a, b, c, a, b, c + 512)  # values partly in place
    assert st == V.VDIT_ERR_INVALID_ARG and "v_out partially overlaps v_in" in msg
    st, msg = qkv(a, b, c, a, b, c, v_gain=a + 4)
    assert st == V.VDIT_ERR_INVALID_ARG and "aligned" in msg
    st, msg = qkv(a, b, c, a, b, c, Hq=64, Hk=64)  # (64 + 64 + 64) x 128 rows of a token > 16384
    assert st == V.VDIT_ERR_UNSUPPORTED and "heads per token" in msg
    st, msg = qkv(None, None, c, None, None, c, Hk=0)
    assert st == V.VDIT_ERR_INVALID_ARG and "n_kv_heads" in msg
    st, msg = qkv(a, b, c, a, b, c, flags=8)
    assert st == V.VDIT_ERR_INVALID_ARG and "flags" in msg
    # the values' flag belongs to vdit_rope_qkv
    st, msg = _status(lib, lib.vdit_rope_qk, a, b, a, b, 1, 100, 12, 12, 128, 0,
                      ctypes.byref(grid), 0, 0, None, None, 1e-6, V.VDIT_ROPE_V_NORM, None)
    assert st == V.VDIT_ERR_INVALID_ARG and "vdit_rope_qkv" in msg


def test_rms_norm_validation_errors_return_before_any_gpu_call(lib):
    fake = 1 << 20  # never dereferenced: validation fails first
    st, msg = _status(lib, lib.vdit_rms_norm, fake, fake, 1, 100, 3, 96, 0, None, 1e-6, None)
    assert st == V.VDIT_ERR_UNSUPPORTED and "head_dim" in msg
    st, msg = _status(lib, lib.vdit_rms_norm, fake, None, 1, 100, 3, 64, 0, None, 1e-6, None)
    assert st == V.VDIT_ERR_INVALID_ARG and "x_out" in msg
    st, msg = _status(lib, lib.vdit_rms_norm, fake, fake + 64, 1, 100, 3, 64, 0, None, 1e-6, None)
    assert st == V.VDIT_ERR_INVALID_ARG and "overlap" in msg
    st, msg = _status(lib, lib.vdit_rms_norm, fake, fake, 1, 100, 3, 64, 0, fake + 4, 1e-6, None)
    assert st == V.VDIT_ERR_INVALID_ARG and "aligned" in msg
    st, msg = _status(lib, lib.vdit_rms_norm, fake, fake, 1, 100, 0, 64, 0, None, 1e-6, None)
    assert st == V.VDIT_ERR_INVALID_ARG and "n_heads" in msg
    st, msg = _status(lib, lib.vdit_rms_norm, fake, fake, 1, 100, 3, 64, 0, None, -1.0, None)
    assert st == V.VDIT_ERR_INVALID_ARG and "eps" in msg


def test_last_error_is_per_thread(lib):
    """vdit_last_error() is thread-local (vdit.h): two threads fail in
    different ways between the same two barriers, and each reads back its own
    message afterwards."""
    import threading
    fake = 1 << 20  # never dereferenced: validation fails first
    calls = {
        "head_dim": lambda: lib.vdit_rms_norm(fake, fake, 1, 100, 3, 96, 0, None, 1e-6, None),
        "eps": lambda: lib.vdit_rms_norm(fake, fake, 1, 100, 3, 64, 0, None, -1.0, None),
    }
    bar = threading.Barrier(2)
    bad = []

    def run(word):
        for _ in range(200):
            st = calls[word]()
            bar.wait()
            bar.wait()
            msg = lib.vdit_last_error().decode()
            if st == V.VDIT_OK or word not in msg:
                bad.append((word, st, msg))

    th = [threading.Thread(target=run, args=(w,)) for w in calls]
    for t in th:
        t.start()
    for t in th:
        t.join()
    assert not bad, bad[:3]


def test_attn_validation_errors(lib):
    a = V.VditAttnArgs()
    a.mode, a.dtype, a.B, a.n_heads, a.n_kv_heads, a.head_dim = 0, 0, 1, 12, 5, 128
    a.Lq = a.Lkv = 64
    a.q, a.k, a.v, a.o = 1 << 20, 2 << 20, 3 << 20, 4 << 20
    st = lib.vdit_attn_fwd(ctypes.byref(a), None)
    assert st == V.VDIT_ERR_INVALID_ARG and "multiple" in lib.vdit_last_error().decode()
    a.n_kv_heads = 12
    a.mode = 3
    a.chunk_tokens = 16
    st = lib.vdit_attn_fwd(ctypes.byref(a), None)
    assert st == V.VDIT_ERR_INVALID_ARG and "state" in lib.vdit_last_error().decode()
    assert lib.vdit_attn_fwd(None, None) == V.VDIT_ERR_INVALID_ARG
    a.mode, a.chunk_tokens = 0, 0
    for bad in (-1.0, float("nan"), float("inf")):
        a.key_norm_max = bad
        st = lib.vdit_attn_fwd(ctypes.byref(a), None)
        assert st == V.VDIT_ERR_INVALID_ARG and "key_norm_max" in lib.vdit_last_error().decode()
    a.key_norm_max = 0.0
    # flags: unknown bits, the ring-only fold flag outside RING and the
    # hybrid-only zero-state flag outside CHUNK_HYBRID
    for flags, word in ((4, "unknown"), (V.VDIT_ATTN_RING_FOLD, "RING"), (V.VDIT_ATTN_STATE_ZERO, "CHUNK_HYBRID")):
        a.flags = flags
        st = lib.vdit_attn_fwd(ctypes.byref(a), None)
        assert st == V.VDIT_ERR_INVALID_ARG and word in lib.vdit_last_error().decode()
    a.flags = 0
    # polynomial feature maps: hybrid only, finite
    coef = (ctypes.c_float * 8)(1, 0.1, 0.01, 0.001, 1, 0.1, 0.01, 0.001)
    a.phi_coef = ctypes.cast(coef, ctypes.c_void_p)
    st = lib.vdit_attn_fwd(ctypes.byref(a), None)
    assert st == V.VDIT_ERR_INVALID_ARG and "CHUNK_HYBRID" in lib.vdit_last_error().decode()
    a.mode, a.chunk_tokens = 3, 16
    a.state_s, a.state_z = 5 << 20, 6 << 20
    coef[5] = float("nan")
    st = lib.vdit_attn_fwd(ctypes.byref(a), None)
    assert st == V.VDIT_ERR_INVALID_ARG and "finite" in lib.vdit_last_error().decode()
    with pytest.raises(ValueError):
        V.vdit_attn_fwd(None, phi_coef=(1.0, 2.0))


def test_workspace_sizes(lib):
    w3 = WL.WORKLOADS[3]
    a = V.VditAttnArgs()
    a.mode, a.dtype, a.B, a.n_heads, a.n_kv_heads, a.head_dim = 1, 0, 1, 10, 10, 128
    a.Lq, a.Lkv, a.n_kv_chunks = 15600, 31200, 2
    o_bytes = 15600 * 10 * 128 * 4
    lse_bytes = 10 * 15600 * 4
    align = lambda x: (x + 255) // 256 * 256
    bound = lambda B, Hk: align(B * Hk * 64 * 4)  # optional key-norm partials (bf16)
    # required running partial + a key-bound run per chunk + one partial per
    # chunk for the one-launch form
    assert V.vdit_attn_workspace_bytes(a) == align(o_bytes) + align(lse_bytes) + align(2 * 10 * 64 * 4) + \
        align(2 * o_bytes) + align(2 * lse_bytes)
    a.dtype = 1  # float32: the fold form only, no key bound
    assert V.vdit_attn_workspace_bytes(a) == align(o_bytes) + align(lse_bytes)
    a.dtype = 0
    a.flags = V.VDIT_ATTN_RING_FOLD  # the fold form on request: no one-launch partials
    assert V.vdit_attn_workspace_bytes(a) == align(o_bytes) + align(lse_bytes) + align(2 * 10 * 64 * 4)
    a.flags = 0
    a.dtype, a.n_kv_chunks = 0, 9  # more chunks than one launch takes: fold form
    assert V.vdit_attn_workspace_bytes(a) == align(o_bytes) + align(lse_bytes) + align(9 * 10 * 64 * 4)
    a.n_kv_chunks = 1
    assert V.vdit_attn_workspace_bytes(a) == bound(1, 10)
    w5 = WL.WORKLOADS[5]
    h = V.VditAttnArgs()
    h.mode, h.dtype, h.B, h.n_heads, h.n_kv_heads, h.head_dim = 3, 0, 1, 24, 24, 128
    h.Lq = h.Lkv = w5.tokens
    h.chunk_tokens = w5.chunk_tokens
    n = V.vdit_attn_workspace_bytes(h)
    nch, ns = 11, 2  # 264 (chunk, head) units -> 2 token splits for ~512 delta workgroups
    expect = align(nch * ns * 24 * 128 * 128 * 4) + align(nch * ns * 24 * 128 * 4) + \
        align(nch * 24 * 128 * 128 * 4) + align(nch * 24 * 128 * 4) + bound(nch, 24)
    assert n == expect
    assert w3.heads == 10
    # FULL on few queries: the optional key-split workspace (256 compute units
    # assumed when no device is present): 2040 queries x 16 heads -> 2 ranges
    f = V.VditAttnArgs()
    f.mode, f.dtype, f.B, f.n_heads, f.n_kv_heads, f.head_dim = 0, 0, 1, 16, 16, 64
    f.Lq, f.Lkv = 2040, 10200
    assert V.vdit_attn_workspace_bytes(f) == bound(1, 16) + align(2 * 2040 * 16 * 64 * 4) + align(2 * 16 * 2040 * 4)
    f.Lq, f.n_heads, f.n_kv_heads, f.head_dim, f.Lkv = 32760, 12, 12, 128, 32760
    assert V.vdit_attn_workspace_bytes(f) == bound(1, 12)
    # several rounds of 128-query workgroups ending on a nearly empty one
    # (14400 queries x 24 heads: 2712 workgroups, 152 in the sixth round of
    # 512): two key ranges
    f.Lq, f.n_heads, f.n_kv_heads, f.head_dim, f.Lkv = 14400, 24, 3, 64, 28800
    assert V.vdit_attn_workspace_bytes(f) == bound(1, 3) + align(2 * 14400 * 24 * 64 * 4) + align(2 * 24 * 14400 * 4)
    # ... but not a call that three workgroups per CU fit in one round
    # (3600 queries x 24 heads: 696 workgroups), nor one with fewer keys
    f.Lq, f.Lkv = 3600, 7200
    assert V.vdit_attn_workspace_bytes(f) == bound(1, 3)
    f.Lq, f.Lkv = 14400, 4096
    assert V.vdit_attn_workspace_bytes(f) == bound(1, 3)
    f.dtype = 1  # float32: neither the bound nor the split
    assert V.vdit_attn_workspace_bytes(f) == 0
    h.head_dim = 96
    with pytest.raises(V.VditError):
        V.vdit_attn_workspace_bytes(h)


def test_binding_fails_loudly_without_library(monkeypatch):
    monkeypatch.setattr(V, "_lib_handle", None)
    monkeypatch.setattr(V, "LIB_PATH", "/nonexistent/libvdit.so")
    with pytest.raises(RuntimeError, match="not built"):
        V.lib()
