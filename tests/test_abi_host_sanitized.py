"""The C ABI's host checks (tests/test_abi.py) run again against a build of the library whose
host code carries AddressSanitizer and UndefinedBehaviorSanitizer (device code as usual), with
clang's ASan runtime preloaded into the test's python: an out-of-bounds access or undefined
behaviour in the host-side argument checking, workspace carving or status reporting aborts the
run.  CPU only (no kernel is launched)."""
import os
import subprocess
import sys

from sparse_moe_ffn_sigmoid_amd import build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_abi_checks_under_host_asan_and_ubsan():
    lib = build.build(host_sanitize=True)
    with open(lib, "rb") as fh:                                         # instrumented host code
        blob = fh.read()
    assert b"__asan_report_load" in blob and b"__ubsan_handle" in blob
    out = subprocess.run([sys.executable, "-c", "import ctypes; ctypes.CDLL(None).__asan_init; print('ok')"],
                         capture_output=True, text=True,
                         env={**os.environ, "LD_PRELOAD": build.asan_runtime(), "ASAN_OPTIONS": "detect_leaks=0"})
    assert out.stdout.strip() == "ok", out.stderr[-2000:]              # the runtime is in the process
    env = {**os.environ, "LD_PRELOAD": build.asan_runtime(), "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1",
           "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1", "MOEFP8_LIB": lib}
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_abi.py"), "-q",
                        "-p", "no:cacheprovider"], capture_output=True, text=True, env=env, cwd=ROOT, timeout=600)
    assert r.returncode == 0, (r.stdout[-3000:], r.stderr[-3000:])
    assert "passed" in r.stdout and "ERROR: AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr
