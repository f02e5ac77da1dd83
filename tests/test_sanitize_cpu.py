"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer, on the CPU.

* The oracle, compiled with clang's sanitizers, runs every pin.
* libq4 with its host code sanitized (the device code is built as usual and never runs
  here) goes through the C-ABI and binding validation suites: every rejected argument,
  the size helpers, the launch record and the status strings.  Calls that pass
  validation reach the HIP runtime, which has no GPU here and fails the launch.
Each runs in a child process with clang's ASan runtime loaded first.  A planted
out-of-bounds write in an oracle copy checks that the sanitizer really reports."""
import os
import subprocess
import sys

import pytest

import oracle
from w4a16_group_wise_q4_amd import _build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN_FLAGS = ("-O1", "-g", "-fno-omit-frame-pointer", "-shared-libsan",
             "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined")
PINS_SCRIPT = """
import sys
sys.path[:0] = [sys.argv[2], sys.argv[3]]
import oracle, pins
o = oracle.Oracle(sys.argv[1])
for check in pins.ALL_CHECKS:
    check(o)
    print("pin", check.__name__, flush=True)
print("all pins ran")
"""


def _env(**extra):
    env = dict(os.environ)
    env["LD_PRELOAD"] = _build.asan_runtime()
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0:exitcode=23"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    env.update(extra)
    return env


def _sanitized_oracle(tmp_path, src=oracle.SOURCE):
    return oracle.compile_source(src, str(tmp_path / "liboracle_san.so"),
                                 include_dir=os.path.dirname(oracle.SOURCE),
                                 compiler=_build.CLANG, extra=SAN_FLAGS)


def _run_pins(lib):
    return subprocess.run([sys.executable, "-c", PINS_SCRIPT, lib, ROOT,
                           os.path.join(ROOT, "tests")],
                          env=_env(), capture_output=True, text=True, timeout=600)


def test_oracle_pins_under_sanitizers(tmp_path):
    res = _run_pins(_sanitized_oracle(tmp_path))
    assert res.returncode == 0 and "all pins ran" in res.stdout, res.stdout[-2000:] + res.stderr[-4000:]


def test_sanitizer_reports_a_planted_overflow(tmp_path):
    src = open(oracle.SOURCE, encoding="utf-8").read()
    old = "float* v = (float*)malloc((size_t)g * sizeof(float));\n    int* q"
    assert src.count(old) == 1
    path = tmp_path / "planted.c"
    path.write_text(src.replace(old, old.replace("(size_t)g *", "(size_t)(g - 1) *")),
                    encoding="utf-8")
    res = _run_pins(_sanitized_oracle(tmp_path, str(path)))
    assert res.returncode != 0 and "heap-buffer-overflow" in res.stderr, res.stderr[-2000:]


def test_c_abi_validation_under_sanitizers(tmp_path):
    lib = _build.build_host_sanitized(str(tmp_path / "libq4_san.so"))
    res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                          "-m", "not gpu", "tests/test_abi_cpu.py",
                          "tests/test_binding_validation.py"],
                         cwd=ROOT, env=_env(Q4_LIBRARY=lib), capture_output=True, text=True,
                         timeout=900)
    tail = res.stdout[-3000:] + res.stderr[-4000:]
    assert res.returncode == 0 and " passed" in res.stdout, tail
    assert "AddressSanitizer" not in res.stderr and "runtime error" not in res.stderr, tail
