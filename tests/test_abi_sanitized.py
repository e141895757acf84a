"""The host-only ABI tests (tests/test_abi.py) against a build whose C ABI
layer (mla_api.cpp: argument checks, workspace layout, dispatch) is compiled
with AddressSanitizer and UndefinedBehaviorSanitizer, undefined behaviour
fatal, run in a child process with the sanitizer runtime preloaded.  CPU
only: every call there fails validation before any HIP work."""
import os
import subprocess
import sys

from mla_latent_kv_nope_amd import build as mla_build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_abi_tests_pass_under_address_and_ub_sanitizers():
    lib = mla_build.build_sanitized(verbose=False)
    runtime = mla_build.sanitizer_runtime()
    env = dict(os.environ)
    env["LD_PRELOAD"] = runtime + (":" + env["LD_PRELOAD"] if env.get("LD_PRELOAD") else "")
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    env["MLA_LIB_PATH"] = lib
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi.py")],
                       env=env, cwd=ROOT, capture_output=True, text=True, timeout=900)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-4000:]
    assert " passed" in out, out[-2000:]
