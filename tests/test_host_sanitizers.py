"""The host side of the library under AddressSanitizer and
UndefinedBehaviorSanitizer: argument validation, workspace arithmetic and
launch set-up, driven by the boundary tests (no GPU involved: every call
there either fails validation or stops at the first device call)."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_boundary_tests_pass_under_host_sanitizers():
    from block_sparse_token_amd import build as BLD

    lib = BLD.build_sanitized()
    runtime = BLD.asan_runtime()
    pre = os.environ.get("LD_PRELOAD", "")
    env = dict(os.environ, UNIPREFILL_LIB=lib,
               # the sanitizer runtime first, anything already preloaded after it
               LD_PRELOAD=runtime + (":" + pre if pre else ""),
               ASAN_OPTIONS="detect_leaks=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_boundary.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    out = r.stdout + r.stderr
    assert "runtime error" not in out, out[-4000:]
    assert "AddressSanitizer" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in r.stdout
