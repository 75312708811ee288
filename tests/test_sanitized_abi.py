"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer
(CPU only): the library's host-arithmetic files are rebuilt with both
sanitizers on their host pass (looped_transformer_decode_amd.build
--sanitize), and the CPU tests of the ABI run against that build in a child
process with the sanitizer runtime preloaded.  Any report aborts the child,
so the test passes only when the run is clean."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.slow
def test_abi_host_code_is_sanitizer_clean():
    from looped_transformer_decode_amd import build as B
    lib = B.build_sanitized()
    env = dict(os.environ,
               LD_PRELOAD=B.sanitizer_runtime(),
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1",
               LLA_LIBRARY=lib)
    cmd = [sys.executable, "-m", "pytest", "-q", "-s", "-p", "no:cacheprovider", "-m", "not gpu",
           os.path.join(ROOT, "tests", "test_abi.py"),
           os.path.join(ROOT, "tests", "test_zz_no_alloc.py")]
    r = subprocess.run(cmd, cwd=ROOT, env=env, stdout=subprocess.PIPE, stderr=subprocess.STDOUT,
                       text=True, timeout=600)
    tail = "\n".join(r.stdout.splitlines()[-40:])
    assert r.returncode == 0, tail
    assert "Sanitizer" not in r.stdout, tail
    assert " passed" in r.stdout, tail
