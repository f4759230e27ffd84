"""The CPU oracle built with AddressSanitizer and UndefinedBehaviorSanitizer
(CPU only).

* Every pin runs clean against the instrumented build: no out-of-bounds
  access, no use of freed memory, no undefined behaviour on any input the
  pins feed it (a report aborts the run).
* Every planted mistake of test_oracle_mutants.py, built the same way, is
  still caught: by a failing pin or by a sanitizer report.

Each run is a child Python process with the sanitizer runtime preloaded (the
interpreter itself is not instrumented; leak checking is off for it)."""
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

from oracle import build as obuild
from tests.test_oracle_mutants import MUTANTS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN_FLAGS = ["-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
             "-fno-omit-frame-pointer"]

DRIVER = """
import sys
import oracle
from tests import pins
bad = pins.failing_pins(oracle.load(sys.argv[1]))
print("FAILING", len(bad))
for name, why in bad:
    print(name, why)
"""


def _asan_runtime():
    if shutil.which("gcc") is None:
        return None
    path = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True,
                          text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


ASAN = _asan_runtime()
pytestmark = pytest.mark.skipif(ASAN is None, reason="gcc's AddressSanitizer runtime not found")


def _build(src, out):
    # The oracle's own flags, then the sanitizers (the later -O1 wins).
    cmd = ["gcc", *obuild.CFLAGS, "-Wno-error", *SAN_FLAGS, src, "-o", out, "-lm"]
    subprocess.run(cmd, check=True, capture_output=True)
    return out


def _run_pins(lib):
    env = dict(os.environ, LD_PRELOAD=ASAN,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    return subprocess.run([sys.executable, "-c", DRIVER, lib], capture_output=True, text=True,
                          cwd=ROOT, env=env, timeout=300)


def test_pins_clean_under_sanitizers(tmp_path):
    lib = _build(obuild.SOURCE, str(tmp_path / "liboracle_san.so"))
    r = _run_pins(lib)
    report = r.stdout + r.stderr
    assert r.returncode == 0, f"sanitized oracle run failed:\n{report[-3000:]}"
    assert "FAILING 0" in r.stdout, f"pins fail on the sanitized build:\n{r.stdout[-2000:]}"
    assert "AddressSanitizer" not in report and "runtime error" not in report, report[-3000:]


def test_mutants_caught_under_sanitizers(tmp_path):
    with open(obuild.SOURCE) as f:
        source = f.read()

    def one(name):
        old, new = MUTANTS[name]
        src = tmp_path / f"m_{name}.c"
        src.write_text(source.replace(old, new))
        lib = _build(str(src), str(tmp_path / f"libm_{name}.so"))
        r = _run_pins(lib)
        caught = r.returncode != 0 or "FAILING 0" not in r.stdout
        return name, caught

    with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        results = list(ex.map(one, sorted(MUTANTS)))
    missed = [n for n, caught in results if not caught]
    assert not missed, f"mutants not caught under sanitizers: {missed}"
