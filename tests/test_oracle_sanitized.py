"""The oracle's pins, run against a build of the oracle with
AddressSanitizer and UndefinedBehaviorSanitizer (gcc, host code only): an
out-of-bounds access, a use of freed memory, a signed overflow, a shift past
the width or a misaligned load anywhere in the oracle aborts the run. The
pins run in a child process with the ASan runtime preloaded (Python itself
is not instrumented) and the oracle routed to the sanitized build."""
import os
import subprocess
import sys

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(os.path.dirname(oracle.__file__), "tq_oracle.c")
PINS = ["test_oracle_converters.py", "test_oracle_fwht_int4.py", "test_oracle_fwht_fp8.py",
        "test_oracle_attention.py", "test_oracle_prefill.py", "test_oracle_dequant.py",
        "test_oracle_kpool.py", "test_oracle_readings.py"]


def _runtime(name):
    path = subprocess.run(["gcc", "-print-file-name=" + name], capture_output=True,
                          text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


def test_oracle_pins_under_asan_and_ubsan(tmp_path):
    asan = _runtime("libasan.so")
    if asan is None:
        pytest.skip("gcc has no AddressSanitizer runtime here")
    so = str(tmp_path / "libtq_oracle_san.so")
    oracle.compile_source(SRC, so, ["-g", "-O1", "-fno-omit-frame-pointer",
                                    "-fsanitize=address,undefined",
                                    "-fno-sanitize-recover=all"])
    env = dict(os.environ)
    env.update(LD_PRELOAD=asan, TQ_ORACLE_LIB=so,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    cmd = [sys.executable, "-m", "pytest", "-q", "-x", "-m", "not gpu", "-p", "no:cacheprovider"]
    cmd += [os.path.join(ROOT, "tests", f) for f in PINS]
    r = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    tail = (r.stdout + r.stderr)[-3000:]
    assert r.returncode == 0, tail
    assert "ERROR: AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, tail
