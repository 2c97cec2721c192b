"""The host code of the C-ABI library (argument checks, workspace sizing,
planning) run under AddressSanitizer and UndefinedBehaviorSanitizer: every
test of test_abi.py again, against libspecattn_hostsan.so, in a child
process that preloads the sanitizer runtime.  Runs without a GPU."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_abi_checks_under_host_asan_and_ubsan():
    from speculative_decoding_attention_amd import build
    lib = build.build_library(host_sanitizers=True)
    env = dict(os.environ,
               LD_PRELOAD=build.asan_runtime(),
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1",
               SPECATTN_TEST_LIB=lib)
    # -s: a sanitizer report goes to the real stderr (a halted child's
    # captured output would be lost)
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-s", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi.py")],
                       env=env, capture_output=True, text=True, timeout=600, cwd=ROOT)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert " passed" in r.stdout
