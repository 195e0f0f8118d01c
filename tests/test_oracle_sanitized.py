"""The oracle's pins under AddressSanitizer and UndefinedBehaviorSanitizer.

moe_oracle.c is rebuilt with -fsanitize=address,undefined (host code only:
the oracle is plain C on the CPU) and the pin suites run again in a child
process that loads that build (MOE_ORACLE_LIB) with the ASan runtime
preloaded.  Any out-of-bounds access, use after free or undefined behaviour
on the pins' inputs aborts the child, and this test fails.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "moe_oracle.c")
PINS = ["tests/test_oracle_pins.py", "tests/test_oracle_bruteforce.py",
        "tests/test_oracle_router_variants.py", "tests/test_oracle_backward.py"]


def _runtime(name):
    p = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True)
    path = p.stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not installed")
def test_oracle_pins_under_asan_and_ubsan(tmp_path):
    asan = _runtime("libasan.so")
    if asan is None:
        pytest.skip("gcc has no ASan runtime")
    lib = str(tmp_path / "libmoe_oracle_asan.so")
    subprocess.run(["gcc", "-O1", "-g", "-fopenmp", "-fPIC", "-shared", "-std=c11",
                    "-fno-fast-math", "-fsanitize=address,undefined", "-fno-omit-frame-pointer",
                    "-fno-sanitize-recover=undefined", "-o", lib, SRC, "-lm"], check=True)
    syms = subprocess.run(["nm", "-D", lib], capture_output=True, text=True).stdout
    assert "__asan_" in syms and "__ubsan_" in syms  # the build is instrumented
    env = dict(os.environ, MOE_ORACLE_LIB=lib, LD_PRELOAD=asan,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    probe = subprocess.run([sys.executable, "-c", "import oracle; print(oracle._load()._name)"],
                           cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    assert probe.returncode == 0, probe.stderr[-2000:]
    assert probe.stdout.strip() == lib  # the pins below run on the sanitized build
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        "-m", "not gpu", *PINS], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=900)
    assert r.returncode == 0, (r.stdout[-3000:] + r.stderr[-3000:])
    assert "passed" in r.stdout and "failed" not in r.stdout
