"""The oracle's pins run against an AddressSanitizer + UndefinedBehaviorSanitizer
build of oracle.c (CPU only, gcc): out-of-bounds accesses, use of freed
memory, signed overflow or invalid shifts anywhere the pins reach fail the
run.  The sanitizer runtimes are preloaded into a child Python process (the
parent is not instrumented)."""
import os
import subprocess
import sys
import tempfile

import pytest

from oracle import build as obuild

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)

SCRIPT = """
import sys
sys.path.insert(0, {tests!r}); sys.path.insert(0, {root!r})
import oracle, pinlib
o = oracle.Oracle({lib!r})
for c in pinlib.ALL_CHECKS:
    c(o)
pinlib.check_codec_exhaustive(o, stride=65537)
print("SANITIZED PINS OK")
"""


def _runtime(name):
    p = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return p if os.path.isabs(p) and os.path.exists(p) else None


@pytest.mark.slow
def test_pins_under_asan_ubsan():
    asan, ubsan = _runtime("libasan.so"), _runtime("libubsan.so")
    if not asan or not ubsan:
        pytest.skip("gcc sanitizer runtimes not installed")
    with tempfile.TemporaryDirectory() as d:
        lib = os.path.join(d, "liboracle_san.so")
        subprocess.run(["gcc", "-O1", "-g", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
                        "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
                        "-fno-omit-frame-pointer", obuild.SRC, "-o", lib, "-lm"], check=True)
        env = dict(os.environ, LD_PRELOAD=f"{asan}:{ubsan}",
                   ASAN_OPTIONS="detect_leaks=0:verify_asan_link_order=0:abort_on_error=1",
                   UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
        r = subprocess.run([sys.executable, "-c", SCRIPT.format(tests=HERE, root=ROOT, lib=lib)], env=env,
                           capture_output=True, text=True, timeout=600)
    assert r.returncode == 0 and "SANITIZED PINS OK" in r.stdout, (r.returncode, r.stdout[-2000:], r.stderr[-4000:])
