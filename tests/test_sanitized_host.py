"""The CPU-side contract tests (argument checks of every C entry point, the
oracle's pins, the input generator) rerun against builds instrumented with
AddressSanitizer and UndefinedBehaviorSanitizer: the library's host code
(device code compiled as usual; no kernel is launched on the CPU) and the
oracle.  Any invalid access or undefined behaviour the runs reach aborts
the subprocess.  The sanitized objects are rebuilt only when a source
changed (about a minute and a half the first time)."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ASAN_RT = "/opt/rocm/llvm/lib/clang/22/lib/linux/libclang_rt.asan-x86_64.so"


@pytest.mark.skipif(not os.path.exists(ASAN_RT), reason="ROCm clang AddressSanitizer runtime not found")
def test_host_code_and_oracle_are_clean_under_address_and_ub_sanitizers():
    sys.path.insert(0, ROOT)
    import oracle
    from top_key_selection_amd import build
    lib = build.build(sanitize=True)
    orc = oracle.build_sanitized(os.path.join(ROOT, "_build", "san"))
    env = dict(os.environ, LD_PRELOAD=ASAN_RT, TKS_LIB=lib, TKS_ORACLE_LIB=orc,
               ASAN_OPTIONS="detect_leaks=0:alloc_dealloc_mismatch=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        "-m", "not gpu", "tests/test_abi.py", "tests/test_oracle_pins.py",
                        "tests/test_inputs_and_golden.py"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert " passed" in out
