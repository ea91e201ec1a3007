"""The oracle's C code under AddressSanitizer and UndefinedBehaviorSanitizer.

The pins of routing, grouping, the experts and the router projection run in
a child process against a copy of the oracle built with
-fsanitize=address,undefined (errors abort, no recovery), the sanitizer
runtimes preloaded into the child.  A copy with one planted out-of-bounds
read must be stopped by the sanitizer, which shows that the instrumented
library is the one the pins exercised.  CPU only.
"""
import os
import shutil
import subprocess
import sys

import pytest

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
PINS = ["test_oracle_route.py", "test_oracle_dispatch.py", "test_oracle_ffn.py", "test_oracle_router.py"]
SAN_FLAGS = ("-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer")


def _runtime(name):
    path = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


def _run_pins(lib, tests):
    env = dict(os.environ)
    env["LD_PRELOAD"] = " ".join(p for p in (_runtime("libasan.so"), _runtime("libubsan.so")) if p)
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    env["TRE_ORACLE_LIB"] = lib
    # -s: the child does not capture its output, so a sanitizer report that
    # ends the process still reaches stderr
    cmd = [sys.executable, "-m", "pytest", "-q", "-x", "-s", "-p", "no:cacheprovider", *tests]
    return subprocess.run(cmd, cwd=HERE, env=env, capture_output=True, text=True, timeout=600)


@pytest.fixture(scope="module")
def sanitizers():
    if shutil.which("gcc") is None or _runtime("libasan.so") is None or _runtime("libubsan.so") is None:
        pytest.skip("gcc's sanitizer runtimes are not installed")


def test_pins_clean_under_sanitizers(sanitizers, tmp_path):
    lib = oracle.build(oracle.SRC_PATH, str(tmp_path / "liboracle_san.so"), SAN_FLAGS)
    r = _run_pins(lib, PINS)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert "passed" in r.stdout


def test_sanitizer_catches_planted_overrun(sanitizers, tmp_path):
    # the routing's normalisation runs one element past its probability array
    src = open(oracle.SRC_PATH).read()
    site = "for (int32_t e = 0; e < E; ++e) prob[e] /= z;"
    assert src.count(site) == 1, "mutation site not found"
    bad = tmp_path / "overread.c"
    bad.write_text(src.replace(site, "for (int32_t e = 0; e <= E; ++e) prob[e] /= z;"))
    lib = oracle.build(str(bad), str(tmp_path / "liboracle_bad.so"), SAN_FLAGS)
    r = _run_pins(lib, ["test_oracle_route.py"])
    assert r.returncode != 0
    assert "AddressSanitizer" in r.stderr or "runtime error" in r.stderr, r.stderr[-3000:]
