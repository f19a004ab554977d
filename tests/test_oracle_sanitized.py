"""The oracle's pins again, with the oracle built under AddressSanitizer and
UndefinedBehaviorSanitizer (CPU only).

A subprocess loads the instrumented build (the ASan runtime preloaded, every
sanitizer report fatal) and runs every oracle pin file; an out-of-bounds
access, a use after free or undefined behaviour anywhere in the C oracle
fails this test.
"""

import os
import subprocess
import sys

import pytest

from oracle import build_oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PINS = ["tests/test_oracle_pins.py", "tests/test_oracle_cost.py", "tests/test_oracle_fp8.py",
        "tests/test_oracle_gated.py", "tests/test_oracle_backward.py"]


@pytest.mark.slow
def test_oracle_pins_under_asan_and_ubsan():
    build_oracle.build(sanitize=True)
    env = build_oracle.sanitizer_env()
    probe = subprocess.run([sys.executable, "-c", "import ctypes; from oracle import oracle; "
                            "print(oracle.lib()._name); print(hasattr(ctypes.CDLL(None), '__asan_init'))"],
                           cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    assert probe.returncode == 0, probe.stderr[-2000:]
    assert probe.stdout.split() == [build_oracle.SAN_LIB, "True"], probe.stdout
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "-m", "not gpu"] + PINS,
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=1200)
    tail = (r.stdout + r.stderr)[-3000:]
    assert r.returncode == 0, tail
    assert "passed" in r.stdout and "ERROR: AddressSanitizer" not in tail and "runtime error" not in tail, tail
