"""The host-side validation cases of test_abi.py, run against a build of the
library whose host code carries AddressSanitizer and UndefinedBehaviorSanitizer.

Every entry point's argument checks run on the host before any launch; this
runs them (no GPU is touched: the cases are the rejection paths, and they run
only where no GPU device node exists) in a child process with the ASan
runtime preloaded and UBSan set to abort on the first report.
"""

import importlib.util
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
NO_GPU = not os.path.exists("/dev/kfd")


def _build_module():
    path = os.path.join(ROOT, "gram_hash_memory_amd", "build.py")
    spec = importlib.util.spec_from_file_location("_engram_build_sanitized", path)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


@pytest.mark.skipif(not NO_GPU, reason="the rejection cases run only without a GPU")
@pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"),
                    reason="needs hipcc")
def test_validation_under_address_and_ub_sanitizers():
    b = _build_module()
    lib = b.build_sanitized()
    runtime = b.sanitizer_runtime()
    assert os.path.exists(runtime), runtime
    env = dict(os.environ, LD_PRELOAD=runtime, ENGRAM_ABI_SANITIZED_LIB=lib,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:exitcode=23",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1:exitcode=24")
    res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                          os.path.join(ROOT, "tests", "test_abi.py"), "-k", "TestValidation"],
                         cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = res.stdout + res.stderr
    assert res.returncode == 0, out[-4000:]
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert " passed" in out and "skipped" not in out.split("\n")[-2], out[-2000:]
