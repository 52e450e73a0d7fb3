"""Build libvdit.so (gfx950) in-tree with hipcc.

``python -m video_diffusion_transformer_rmsnorm_amd.build`` compiles every
source under ``csrc/`` for gfx950 and links ``libvdit.so`` next to this file.
Objects go to ``_build/`` at the repository root.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libvdit.so")
ARCH = "gfx950"

SOURCES = ["abi.cpp", "rope_qk.hip", "lse_merge.hip", "attn_mfma.hip", "attn_valu.hip", "hybrid_state.hip",
           "key_bound.hip", "noalloc.hip"]

# Packed float32 VALU forms are disabled on purpose: the compiler otherwise
# forms them from ordinary float code.
COMMON = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]


def hipcc() -> str:
    for c in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def _compile(src: str, extra, tag: str = "") -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + tag + ".o")
    cmd = [hipcc(), *COMMON, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


DEBUG_SYNC_LIB = os.path.join(PKG, "libvdit_debugsync.so")


def build(verbose: bool = False, extra=(), lib: str = LIB, tag: str = "") -> str:
    """Compile all sources and link libvdit.so (or `lib`, objects suffixed
    `tag`); returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 4)) as ex:
        objs = list(ex.map(lambda s: _compile(s, list(extra), tag), SOURCES))
    tmp = lib + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)
    if verbose:
        print(f"built {lib}")
    return lib


def build_debug_sync(verbose: bool = False) -> str:
    """The self-check build of the library (VDIT_DEBUG_SYNC=1: every pipeline
    stage of the attention kernel ends on a full wait and a barrier), which
    the GPU tests compare bit for bit with libvdit.so."""
    return build(verbose, extra=("-DVDIT_DEBUG_SYNC=1",), lib=DEBUG_SYNC_LIB, tag=".debugsync")


PROBES_SRC = os.path.join(CSRC, "probes", "mfma_peak.hip")
PROBES_LIB = os.path.join(PKG, "libvdit_probes.so")


def build_probes(verbose: bool = False) -> str:
    """Compile the measurement probes the benchmark uses (not part of the
    library's ABI) into libvdit_probes.so; returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    tmp = PROBES_LIB + ".tmp"
    cmd = [hipcc(), *COMMON, "-shared", PROBES_SRC, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, PROBES_LIB)
    if verbose:
        print(f"built {PROBES_LIB}")
    return PROBES_LIB


CONSUMER_SRC = os.path.join(ROOT, "tests", "host", "c_consumer.c")
CONSUMER = os.path.join(ROOT, "tests", "host", "c_consumer")


def build_consumer(verbose: bool = False) -> str:
    """Compile the plain C test program that links libvdit.so (the C ABI
    used without Python); returns its path.  The library must be built."""
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        raise RuntimeError("no C compiler found")
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    rel = os.path.relpath(PKG, os.path.dirname(CONSUMER))
    cmd = [cc, "-std=c99", "-O2", "-Wall", "-Werror", "-D__HIP_PLATFORM_AMD__", "-I", INCLUDE,
           "-I", os.path.join(rocm, "include"), CONSUMER_SRC, "-o", CONSUMER, "-L", PKG, "-lvdit",
           "-L", os.path.join(rocm, "lib"), "-lamdhip64", f"-Wl,-rpath,$ORIGIN/{rel}",
           f"-Wl,-rpath,{os.path.join(rocm, 'lib')}"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    if verbose:
        print(f"built {CONSUMER}")
    return CONSUMER


if __name__ == "__main__":
    build(verbose=True, extra=sys.argv[1:])
    build_debug_sync(verbose=True)
    build_probes(verbose=True)
    build_consumer(verbose=True)
