"""The oracle (plain C) under AddressSanitizer and UndefinedBehaviorSanitizer:
oracle.c is built with -fsanitize=address,undefined (no recovery) and the
oracle's own CPU pin tests run against that build in a child process.  Any
out-of-bounds access, use after free or undefined operation in the oracle
aborts the child with a sanitizer report."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ORACLE_TESTS = ["test_oracle_dispatch.py", "test_oracle_combine.py", "test_oracle_partial.py",
                "test_oracle_fixed_slot.py", "test_oracle_codecs.py", "test_oracle_threads.py"]


def _runtime(name: str) -> str:
    path = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True,
                          text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else ""


def test_oracle_under_asan_and_ubsan(tmp_path):
    asan = _runtime("libasan.so")
    if not asan:
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    lib = str(tmp_path / "liboracle_san.so")
    subprocess.run(["gcc", "-O1", "-g", "-fno-omit-frame-pointer", "-ffp-contract=off",
                    "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fPIC",
                    "-shared", "-o", lib, os.path.join(ROOT, "oracle", "oracle.c"), "-lm"],
                   check=True)
    env = dict(os.environ)
    env.update(ORACLE_LIBRARY=lib, LD_PRELOAD=asan,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:allocator_may_return_null=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    tests = [os.path.join(ROOT, "tests", t) for t in ORACLE_TESTS]
    res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-s", "-x", "-m", "not gpu",
                          "-p", "no:cacheprovider"] + tests,
                         cwd=ROOT, env=env, capture_output=True, text=True, timeout=1200)
    out = res.stdout + res.stderr
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert res.returncode == 0, out[-4000:]
    assert " passed" in res.stdout
