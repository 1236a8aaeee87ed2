"""The C ABI's host layer under AddressSanitizer and UndefinedBehaviorSanitizer:
abi.cpp (argument validation, workspace views, kernel choice) is rebuilt by
g++ with -fsanitize=address,undefined, linked with the same gfx950 kernel
objects, and the whole CPU ABI suite (tests/test_abi_cpu.py) runs against it
in a child process with gcc's ASan runtime preloaded. Any invalid read or
write, or any undefined behaviour, in the validation paths aborts that
process. No GPU is involved: every call in that suite returns before its
first HIP call."""

import os
import subprocess
import sys

from megatron_sharded_linears_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_abi_suite_under_asan_and_ubsan():
    lib = B.build_sanitized(verbose=False)
    env = dict(os.environ)
    env.update({"LD_PRELOAD": B.asan_runtime(), "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1",
                "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1", "TPSHARD_LIB": lib,
                "TPSHARD_EXPECT_SANITIZED": "1"})
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi_cpu.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert "passed" in r.stdout and "failed" not in r.stdout, r.stdout[-2000:]
