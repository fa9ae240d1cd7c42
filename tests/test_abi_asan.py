"""The C-ABI's host code under AddressSanitizer: the CPU tests of test_abi_cpu.py
run in a child process against libnbattn_asan.so (nbattn_host.cpp built with
host-side -fsanitize=address, device code unchanged), with the ASan runtime
preloaded.  Any out-of-bounds access or use-after-free in the argument checks,
the chunk and owner tables or the workspace arithmetic aborts the child."""
import os
import subprocess
import sys

import pytest

from sliding_window_attention_fold_amd import build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_abi_checks_under_host_asan():
    if not os.path.exists(build.ASAN_LIB):
        pytest.skip("libnbattn_asan.so is not built (build.build_asan(), run by __graft_entry__.build())")
    env = dict(os.environ)
    env["LD_PRELOAD"] = build.asan_runtime()
    env["NBATTN_LIB"] = build.ASAN_LIB
    # Python itself is not instrumented: leak reports would be about the interpreter
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1"
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi_cpu.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert "AddressSanitizer" not in r.stderr, r.stderr[-3000:]
    assert " passed" in r.stdout
