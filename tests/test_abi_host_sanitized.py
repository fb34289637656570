"""The host-only ABI checks (test_abi_host.py) rerun against a build whose
argument validation and block-pool code carry AddressSanitizer and
UndefinedBehaviorSanitizer on their host pass, in a child process with the
sanitizer runtime preloaded.  Any out-of-bounds access, use after free or
undefined behaviour in that host code aborts the child and fails this test.
No GPU is needed: every call there is rejected before a launch, or is a size
query or a host-side block-pool operation."""

import os
import shutil
import subprocess
import sys

import pytest

from long_context_compressed_csa_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_abi_host_checks_under_host_sanitizers():
    if shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"):
        pytest.skip("no hipcc: the sanitizer build needs the ROCm toolchain")
    rt = B.sanitizer_runtime()
    if rt is None:
        pytest.skip("no AddressSanitizer runtime in the ROCm toolchain")
    if not all(os.path.exists(os.path.join(B.BUILD, f + ".o")) for f in ("attend.hip", "indexer.hip")):
        pytest.skip("the regular build's objects are missing (build the library first)")
    lib = B.build_host_sanitized()
    env = dict(os.environ)
    env["CSA_LIBRARY"] = lib
    # the sanitizer runtime goes first; whatever was preloaded before stays
    env["LD_PRELOAD"] = rt + (":" + env["LD_PRELOAD"] if env.get("LD_PRELOAD") else "")
    # the interpreter itself is not instrumented and keeps memory until exit
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    p = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_abi_host.py"), "-q", "-x",
                        "-p", "no:cacheprovider", "-m", "not gpu"], cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=600)
    tail = (p.stdout + p.stderr)[-4000:]
    assert p.returncode == 0, tail
    assert "passed" in p.stdout and "ERROR: AddressSanitizer" not in tail and "runtime error" not in tail, tail
