"""The host layer under AddressSanitizer and UndefinedBehaviorSanitizer: the
library is built with its host code sanitized (build --sanitize), and the
whole C-ABI suite (tests/test_abi.py: every rejection path, the plan and
workspace queries) runs against it in a child process with the ASan runtime
preloaded.  Any sanitizer report fails the run (UBSan halts on error)."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


@pytest.mark.skipif(not os.path.exists(HIPCC) or shutil.which("g++") is None, reason="needs hipcc")
def test_abi_suite_is_clean_under_asan_and_ubsan():
    sys.path.insert(0, ROOT)
    from paged_gqa_decode_lgm_amd import build

    lib = build.build(sanitize=True)
    rt = subprocess.run([HIPCC, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True,
                        text=True).stdout.strip()
    assert os.path.exists(rt), rt
    env = dict(os.environ, LGM_LIBRARY=lib, LD_PRELOAD=rt, ASAN_OPTIONS="detect_leaks=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_abi.py"), "-q",
                        "-p", "no:cacheprovider", "-p", "no:xdist"], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-4000:]
