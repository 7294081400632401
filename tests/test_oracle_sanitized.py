"""The oracle's pins against an AddressSanitizer + UndefinedBehaviorSanitizer build of
oracle.c, on the CPU.

The sanitized library is compiled with gcc into a temporary directory and loaded in a
child Python process that has the sanitizer runtimes preloaded (a sanitized shared
object cannot be loaded into an interpreter that was started without them). Any
out-of-bounds access, use after free or undefined operation in the oracle while the
pins run ends that process with an error, and the test fails with its report.
"""
import os
import shutil
import subprocess
import sys

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")


def runtime(name):
    path = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


def test_pins_under_asan_and_ubsan(tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    asan, ubsan = runtime("libasan.so"), runtime("libubsan.so")
    if not asan or not ubsan:
        pytest.skip("sanitizer runtimes not installed")
    so = tmp_path / "oracle_sanitized.so"
    flags = [f for f in oracle.CFLAGS if f != "-O2"] + ["-O1", "-g", "-fno-omit-frame-pointer",
                                                         "-fsanitize=address,undefined",
                                                         "-fno-sanitize-recover=undefined"]
    subprocess.run(["gcc", *flags, SRC, "-o", str(so), "-lm"], check=True)
    script = (
        "import sys\n"
        f"sys.path.insert(0, {ROOT!r})\n"
        "import oracle\n"
        "from tests import oracle_pins\n"
        f"o = oracle.Oracle(oracle.load({str(so)!r}))\n"
        "for pin in oracle_pins.ALL_PINS:\n"
        "    pin(o)\n"
        "print('pins passed:', len(oracle_pins.ALL_PINS))\n"
    )
    env = dict(os.environ, LD_PRELOAD=f"{asan}:{ubsan}",
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-c", script], env=env, capture_output=True, text=True, timeout=900,
                       cwd=ROOT)
    assert r.returncode == 0 and "pins passed:" in r.stdout, (r.stdout[-2000:], r.stderr[-4000:])
    assert "runtime error" not in r.stderr, r.stderr[-4000:]
