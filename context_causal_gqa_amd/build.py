"""Build libpcpattn.so (the C-ABI library) in-tree for gfx950.

Usage: python -m context_causal_gqa_amd.build [--verbose]
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libpcpattn.so")
SOURCES = ["pcp_plan.cpp", "pcp_sched.cpp", "pcp_attn_kernels.hip", "pcp_attn_fp8.hip",
           "pcp_cache_write.hip"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # Keep hipcc from forming packed fp32 (v_pk_*_f32) instructions.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm not installed?)")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(
        line for line in (res.stdout + res.stderr).splitlines()
        if "packed-fp32-ops" not in line  # the host pass does not know the feature
    )
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + out)
    if verbose and out.strip():
        print(out)


def _check_loads(path: str) -> None:
    """dlopen the linked library with every symbol resolved now: a launch stub
    that a compiler pass failed to emit shows up here, not at first use."""
    import ctypes

    try:
        ctypes.CDLL(path, mode=os.RTLD_NOW)
    except OSError as e:
        raise RuntimeError("linked library does not load: %s" % e) from None


def build(verbose: bool = False) -> str:
    """Compile every source to an object (in parallel), link them into LIB
    (atomically replaced). Returns the path."""
    from concurrent.futures import ThreadPoolExecutor

    tag = "%d" % os.getpid()
    objs = [os.path.join(CSRC, s + ".%s.o" % tag) for s in SOURCES]
    compile_flags = [f for f in HIPCC_FLAGS if f != "-shared"]
    cmds = [[hipcc()] + compile_flags + ["-I" + INCLUDE, "-c", os.path.join(CSRC, s), "-o", o]
            for s, o in zip(SOURCES, objs)]
    tmp = LIB + ".tmp" + tag
    try:
        with ThreadPoolExecutor(max_workers=min(len(cmds), 8)) as ex:
            list(ex.map(lambda c: _run(c, verbose), cmds))
        _run([hipcc()] + HIPCC_FLAGS + objs + ["-o", tmp], verbose)
        _check_loads(tmp)
        os.replace(tmp, LIB)
    finally:
        for f in objs + [tmp]:
            if os.path.exists(f):
                os.remove(f)
    return LIB


if __name__ == "__main__":
    print(build(verbose="--verbose" in sys.argv))
