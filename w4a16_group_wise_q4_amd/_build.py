"""Build libq4.so in-tree with hipcc for gfx950."""
from __future__ import annotations

import glob
import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIBRARY = os.path.join(PKG, "libq4.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 VALU forms are kept out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
]


LINK_FLAGS = [f"--offload-arch={ARCH}", "-fPIC", "-shared"]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip"))) + [os.path.join(CSRC, "q4_abi.cpp")]


def _run(cmd):
    res = subprocess.run(cmd, capture_output=True, text=True)
    return res.returncode, res.stdout + res.stderr


def build(verbose: bool = False) -> str:
    """Compile every kernel and the C ABI into one shared library (always rebuilds).

    Each source compiles to its own object in parallel (the group-size instantiations of
    the decode tile kernel live in separate files for this), then one link."""
    from concurrent.futures import ThreadPoolExecutor

    objdir = os.path.join(PKG, "_build_obj")
    os.makedirs(objdir, exist_ok=True)
    srcs = sources()
    objs = [os.path.join(objdir, os.path.basename(src) + ".%d.o" % os.getpid()) for src in srcs]
    cmds = [[HIPCC, *FLAGS, "-c", "-I", INCLUDE, "-I", CSRC, src, "-o", obj] for src, obj in zip(srcs, objs)]
    workers = max(1, min(len(cmds), os.cpu_count() or 1, 16))
    with ThreadPoolExecutor(max_workers=workers) as pool:
        results = list(pool.map(_run, cmds))
    logs = []
    try:
        for src, (rc, out) in zip(srcs, results):
            if rc != 0:
                raise RuntimeError("hipcc failed on %s:\n%s" % (os.path.basename(src), out))
            logs.append(out)
        tmp = LIBRARY + ".tmp%d" % os.getpid()
        rc, out = _run([HIPCC, *LINK_FLAGS, *objs, "-o", tmp])
        if rc != 0:
            raise RuntimeError("hipcc failed linking libq4:\n" + out)
        logs.append(out)
    finally:
        for obj in objs:
            if os.path.exists(obj):
                os.remove(obj)
    if verbose:
        noise = "packed-fp32-ops"
        for line in "\n".join(logs).splitlines():
            if noise not in line:
                print(line)
    os.replace(tmp, LIBRARY)
    return LIBRARY
