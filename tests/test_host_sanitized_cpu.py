"""The host side of the C ABI under AddressSanitizer and UBSan: the library
is rebuilt with sanitized host code (device code unchanged) and the whole of
tests/test_abi_cpu.py (symbol exports, capacities, every entry point's
argument and size checks) runs against it in a child process with the
sanitizer runtime preloaded.  Any report fails the run."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _have_hipcc():
    return any(os.path.exists(p) for p in ("/opt/rocm/bin/hipcc",)) or shutil.which("hipcc")


@pytest.mark.skipif(not _have_hipcc(), reason="hipcc is needed to build the sanitized library")
def test_abi_checks_are_clean_under_asan_and_ubsan():
    sys.path.insert(0, ROOT)
    from grouped_gemm_route_amd import build_host_sanitized as S

    lib = S.build(verbose=False)
    env = dict(os.environ)
    env["LD_PRELOAD"] = S.runtime()
    # the interpreter itself is not instrumented: its allocations are not
    # tracked for leaks; every report in the library's code is fatal
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    code = ("import sys; sys.path.insert(0, %r); "
            "import grouped_gemm_route_amd.binding as B; B.LIB_PATH = %r; "
            "assert B.load_library()._name == %r; import pytest; "
            "sys.exit(pytest.main([%r, '-q', '-p', 'no:cacheprovider']))"
            % (ROOT, lib, lib, os.path.join(ROOT, "tests", "test_abi_cpu.py")))
    r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True,
                       timeout=600, cwd=ROOT)
    report = r.stdout + r.stderr
    assert "AddressSanitizer" not in report and "runtime error" not in report, report[-4000:]
    assert r.returncode == 0, report[-4000:]
    assert " passed" in r.stdout
