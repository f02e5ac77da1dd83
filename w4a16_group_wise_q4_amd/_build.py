"""Build libq4.so in-tree with hipcc for gfx950."""
from __future__ import annotations

import glob
import hashlib
import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIBRARY = os.path.join(PKG, "libq4.so")
# the probes the benchmark measures ceilings and costs with (not part of the C ABI): the
# streaming read and the cross-workgroup join of partial sums
PROBE_SOURCES = [os.path.join(PKG, "probe", "read_probe.hip"), os.path.join(PKG, "probe", "join_probe.hip")]
PROBE_LIBRARY = os.path.join(PKG, "libq4probe.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 VALU forms are kept out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
]


LINK_FLAGS = [f"--offload-arch={ARCH}", "-fPIC", "-shared"]

# A debug build for the CPU: AddressSanitizer and UndefinedBehaviorSanitizer on the host
# code only (argument validation, launch shapes, the launch record); the device code is
# compiled as usual and nothing of it is instrumented.
HOST_SANITIZE = ["-Xarch_host", "-fsanitize=address",
                 "-Xarch_host", "-fsanitize=undefined",
                 "-Xarch_host", "-fno-sanitize-recover=undefined",
                 "-Xarch_host", "-fno-omit-frame-pointer"]
CLANG = os.path.join(os.path.dirname(os.path.realpath(HIPCC)), "..", "llvm", "bin", "clang")


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip"))) + [os.path.join(CSRC, "q4_abi.cpp")]


def digested_files():
    """Every file the library is built from: the kernel sources, their headers, the C ABI
    and include/q4.h."""
    files = []
    for pat in ("*.hip", "*.h", "*.cpp"):
        files += glob.glob(os.path.join(CSRC, pat))
    files += glob.glob(os.path.join(INCLUDE, "*.h"))
    return sorted(files, key=lambda f: os.path.relpath(f, ROOT))


def source_digest() -> str:
    """First 16 hex digits of a SHA-256 over (relative path, contents) of every source file;
    compiled into the library and returned by q4_source_digest()."""
    h = hashlib.sha256()
    for f in digested_files():
        h.update(os.path.relpath(f, ROOT).replace(os.sep, "/").encode())
        h.update(b"\0")
        with open(f, "rb") as fh:
            h.update(fh.read())
        h.update(b"\0")
    return h.hexdigest()[:16]


def _run(cmd):
    res = subprocess.run(cmd, capture_output=True, text=True)
    return res.returncode, res.stdout + res.stderr


def _compile_link(flags, link_flags, out, verbose=False, probe=True):
    """Compile every source to its own object in parallel (the group-size instantiations
    of the decode tile kernel live in separate files for this), then one link into out;
    with probe, the read probe library is built in the same pool."""
    from concurrent.futures import ThreadPoolExecutor

    objdir = os.path.join(PKG, "_build_obj")
    os.makedirs(objdir, exist_ok=True)
    srcs = sources()
    tag = "%d.%s" % (os.getpid(), os.path.basename(out))
    objs = [os.path.join(objdir, os.path.basename(src) + ".%s.o" % tag) for src in srcs]
    digest = f'-DQ4_SOURCE_DIGEST="{source_digest()}"'
    cmds = [[HIPCC, *flags, digest, "-c", "-I", INCLUDE, "-I", CSRC, src, "-o", obj]
            for src, obj in zip(srcs, objs)]
    probe_tmp = PROBE_LIBRARY + ".tmp%d" % os.getpid()
    if probe:
        cmds.append([HIPCC, *FLAGS, *LINK_FLAGS[1:], *PROBE_SOURCES, "-o", probe_tmp])
    workers = max(1, min(len(cmds), os.cpu_count() or 1, 16))
    with ThreadPoolExecutor(max_workers=workers) as pool:
        results = list(pool.map(_run, cmds))
    logs = []
    tmp = out + ".tmp%d" % os.getpid()
    try:
        labels = [os.path.basename(src) for src in srcs]
        labels.append("the probes (%s)" % ", ".join(os.path.basename(f) for f in PROBE_SOURCES))
        for label, (rc, text) in zip(labels, results):
            if rc != 0:
                raise RuntimeError("hipcc failed on %s:\n%s" % (label, text))
            logs.append(text)
        rc, text = _run([HIPCC, *link_flags, *objs, "-o", tmp])
        if rc != 0:
            raise RuntimeError("hipcc failed linking libq4:\n" + text)
        logs.append(text)
    finally:
        for obj in objs:
            if os.path.exists(obj):
                os.remove(obj)
    if verbose:
        noise = "packed-fp32-ops"
        for line in "\n".join(logs).splitlines():
            if noise not in line:
                print(line)
    os.replace(tmp, out)
    if probe:
        os.replace(probe_tmp, PROBE_LIBRARY)
    return out


def build(verbose: bool = False) -> str:
    """Compile every kernel and the C ABI into one shared library (always rebuilds), and
    the read probe beside it."""
    return _compile_link(FLAGS, LINK_FLAGS, LIBRARY, verbose=verbose)


def build_host_sanitized(out: str) -> str:
    """libq4 with its host code under AddressSanitizer and UndefinedBehaviorSanitizer, for
    exercising the C ABI on a CPU.  The process that loads it must have clang's ASan
    runtime loaded first (LD_PRELOAD=asan_runtime()); load it through the binding by
    setting Q4_LIBRARY to out.  Carries the same source digest as build()."""
    flags = [f for f in FLAGS if f != "-O3"] + ["-O1", "-g", *HOST_SANITIZE]
    link = [*LINK_FLAGS, "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-shared-libsan"]
    return _compile_link(flags, link, out, probe=False)


def asan_runtime() -> str:
    """Path of clang's shared ASan runtime (which also carries the UBSan handlers)."""
    res = subprocess.run([CLANG, "-print-file-name=libclang_rt.asan-x86_64.so"],
                         capture_output=True, text=True, check=True)
    path = res.stdout.strip()
    if not os.path.isabs(path) or not os.path.exists(path):
        raise RuntimeError("clang's ASan runtime was not found: " + path)
    return path
