"""The host-side tests (argument checks, binding checks, library loading)
against a build of the library whose host code carries AddressSanitizer and
UndefinedBehaviorSanitizer.  The sanitized library is loaded in a child
Python with the sanitizer runtime preloaded; any report fails the test.  No
GPU is needed: every call these tests make is rejected on the host, or fails
cleanly where no device is present."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HOST_TESTS = ["tests/test_boundary_cpu.py", "tests/test_binding_checks_cpu.py"]


def test_host_entry_points_under_asan_and_ubsan():
    from mla_latent_cache_absorbed_amd import build as b
    if not shutil.which(b.HIPCC) and not os.path.exists(b.HIPCC):
        pytest.skip("hipcc is not installed")
    rt = b.sanitizer_runtime()
    if not rt:
        pytest.skip("the compiler's AddressSanitizer runtime is not installed")
    lib = b.build_host_sanitized()
    code = (
        "import sys\n"
        f"sys.path.insert(0, {ROOT!r})\n"
        "import mla_latent_cache_absorbed_amd._lib as L\n"
        f"L.LIB_PATH = {lib!r}\n"
        "import pytest\n"
        f"sys.exit(pytest.main(['-q', '-p', 'no:cacheprovider', *{HOST_TESTS!r}]))\n"
    )
    env = dict(os.environ)
    env["LD_PRELOAD"] = rt
    # the interpreter itself leaks by design; halt at the first report
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1:abort_on_error=0"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=600)
    out = r.stdout + r.stderr
    assert "runtime error" not in out and "AddressSanitizer" not in out.replace(
        "AddressSanitizer: failed to intercept", ""), out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in r.stdout, out[-4000:]
