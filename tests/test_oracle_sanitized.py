"""The oracle under AddressSanitizer and UndefinedBehaviorSanitizer: oracle.c compiled with
-fsanitize=address,undefined (errors fatal), every pin run against that build in a child
process with the ASan runtime preloaded into the interpreter.  An out-of-bounds read or write, a
use of freed memory, a signed overflow or a misaligned access anywhere the pins reach ends the
child with the sanitizer's report.  Host code only; nothing here touches a GPU."""
import os
import shutil
import subprocess
import sys

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g"]


def _runtime(name):
    p = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return p if os.path.isabs(p) and os.path.exists(p) else None


@pytest.mark.skipif(shutil.which("gcc") is None or _runtime("libasan.so") is None,
                    reason="gcc with the ASan runtime is not installed")
def test_pins_under_address_and_ub_sanitizers(tmp_path):
    lib = oracle.build(oracle.SRC, str(tmp_path / "liboracle_san.so"), extra_flags=SAN_FLAGS)
    env = dict(os.environ)
    env["LD_PRELOAD"] = _runtime("libasan.so")
    # the interpreter itself is not instrumented: its allocations are not leaks of the oracle
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0:exitcode=99"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    env["OMP_NUM_THREADS"] = "4"
    r = subprocess.run([sys.executable, os.path.join(ROOT, "tests", "oracle_pins.py"), lib],
                       capture_output=True, text=True, cwd=ROOT, env=env, timeout=900)
    report = r.stdout + r.stderr
    assert "AddressSanitizer" not in report and "runtime error" not in report, report[-4000:]
    assert r.returncode == 0, report[-4000:]


def test_sanitized_build_catches_a_planted_overrun(tmp_path):
    """The set-up is live: an oracle with a planted one-past-the-end read is stopped by ASan."""
    if shutil.which("gcc") is None or _runtime("libasan.so") is None:
        pytest.skip("gcc with the ASan runtime is not installed")
    src = open(oracle.SRC).read()
    old = "for (int d = 0; d < head_dim; ++d)\n                acc +="
    assert src.count(old) == 1
    mut = tmp_path / "oracle_overrun.c"
    mut.write_text(src.replace(old, "for (int d = 0; d <= head_dim; ++d)\n                acc +="))
    lib = oracle.build(str(mut), str(tmp_path / "liboracle_overrun.so"), extra_flags=SAN_FLAGS)
    code = ("import sys, numpy as np, oracle\n"
            "o = oracle.Oracle(sys.argv[1])\n"
            "f = np.ones((3, 1, 8), np.float32)\n"
            "i = np.array([2], np.int32)\n"
            "o.sddmm(i, i, f, f)\n")
    env = dict(os.environ)
    env["LD_PRELOAD"] = _runtime("libasan.so")
    env["ASAN_OPTIONS"] = "detect_leaks=0:exitcode=99"
    r = subprocess.run([sys.executable, "-c", code, lib], capture_output=True, text=True, cwd=ROOT, env=env,
                       timeout=300)
    assert r.returncode != 0 and "AddressSanitizer" in r.stderr, (r.returncode, r.stderr[-2000:])
