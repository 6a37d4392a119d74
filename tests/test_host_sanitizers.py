"""The host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

abi.cpp (argument validation, workspace planning and dispatch) and oracle.c are rebuilt at
-O0 -g with -fsanitize=address,undefined, and the C-ABI and oracle test files run against those
builds in a child process with the ASan runtime preloaded. Any sanitizer report aborts the
child, and so fails this test. Device code is not sanitized (no GPU runs here)."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _asan_runtime():
    if not shutil.which("gcc") or not shutil.which("g++"):
        return None
    out = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True)
    path = out.stdout.strip()
    return path if out.returncode == 0 and os.path.isabs(path) and os.path.exists(path) else None


def test_host_code_under_sanitizers(tmp_path):
    runtime = _asan_runtime()
    if runtime is None:
        pytest.skip("gcc's AddressSanitizer runtime is not available")
    from normalization_reductions_amd import build as nb

    lib, orc = nb.build_host_asan(str(tmp_path))
    env = dict(os.environ)
    env.update({
        "LD_PRELOAD": runtime,
        "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1:halt_on_error=1",
        "UBSAN_OPTIONS": "halt_on_error=1:abort_on_error=1:print_stacktrace=1",
        "NORMRED_LIB": lib,
        "NORMRED_ORACLE_LIB": orc,
    })
    # the child first proves that it loaded the sanitized builds, then runs the two test files
    probe = ("import normalization_reductions_amd._lib as L, oracle as O; L.load(); O._load();"
             "maps = open('/proc/self/maps').read();"
             "assert %r in maps and %r in maps, 'sanitized builds not loaded'; print('loaded')"
             % (lib, orc))
    res = subprocess.run([sys.executable, "-c", probe], cwd=ROOT, env=env, capture_output=True,
                         text=True, timeout=300)
    assert res.returncode == 0 and "loaded" in res.stdout, res.stdout + res.stderr
    res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-m", "not gpu",
                          "-p", "no:cacheprovider", "tests/test_abi_cpu.py",
                          "tests/test_oracle_pins.py"],
                         cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    tail = (res.stdout + res.stderr)[-4000:]
    assert res.returncode == 0, tail
    assert "ERROR: AddressSanitizer" not in tail and "runtime error:" not in tail, tail
