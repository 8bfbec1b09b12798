"""The oracle's pin battery, run once more with the oracle built under
AddressSanitizer and UndefinedBehaviorSanitizer (gcc, host code only).

The checker reads caller buffers through plain indices; a read past a mask,
a bias, a block table or a cache would not change a pin's verdict by itself,
so the sanitized build is what shows that every read stays inside the
buffers the pins hand it.  The battery runs in a child process with the
sanitizer runtime preloaded (Python itself is not instrumented)."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")

RUNNER = r"""
import sys
sys.path.insert(0, {root!r})
sys.path.insert(0, {tests!r})
import oracle
oracle._lib = oracle.bind({lib!r})
import pytest
sys.exit(pytest.main(["-x", "-q", "-s", "-p", "no:cacheprovider", "-o", "addopts=",
                      {pins!r}, {breadth!r}, "-k", "not exhaustive"]))
"""


def _runtime(name):
    path = subprocess.run(["gcc", "-print-file-name=" + name], capture_output=True, text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


def test_pin_battery_under_address_and_undefined_sanitizers(tmp_path):
    asan = _runtime("libasan.so")
    if asan is None:
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    lib = str(tmp_path / "liboracle_asan.so")
    subprocess.check_call(["gcc", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                           "-fno-sanitize-recover=all", "-fopenmp", "-shared", "-fPIC", "-std=c11", SRC, "-o", lib,
                           "-lm"])
    tests = os.path.join(ROOT, "tests")
    script = RUNNER.format(root=ROOT, tests=tests, lib=lib, pins=os.path.join(tests, "test_oracle_pins.py"),
                           breadth=os.path.join(tests, "test_oracle_sfa_breadth.py"))
    env = dict(os.environ)
    # the sanitizer runtime must come first; anything already preloaded stays
    env["LD_PRELOAD"] = asan + (":" + env["LD_PRELOAD"] if env.get("LD_PRELOAD") else "")
    # Python's own allocations are not instrumented and are never freed at exit
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    env["OMP_NUM_THREADS"] = "4"
    # -s above: the sanitizer reports on stderr, which pytest would otherwise capture
    r = subprocess.run([sys.executable, "-c", script], env=env, capture_output=True, text=True, timeout=900)
    tail = (r.stdout[-3000:] + "\n" + r.stderr[-6000:])
    assert r.returncode == 0, tail
    assert "ERROR: AddressSanitizer" not in r.stderr and "runtime error:" not in r.stderr, tail
    assert " passed" in r.stdout, tail
