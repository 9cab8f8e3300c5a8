"""The host code of the C ABI under AddressSanitizer: the library's host pass is rebuilt with
ASan (device code unchanged) and every host-side test of the ABI (symbol exports, argument
checks of every entry point, workspace arithmetic, enum values) runs against it in a child
process that preloads the ASan runtime. A negative control built and loaded the same way
reads one element past a heap array and must be reported, so a silent run means the
instrumentation was active and found nothing. CPU only."""
import os
import subprocess
import sys
import textwrap

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def asan():
    from dropless_mixture_experts_device_amd import build_asan
    rt = build_asan.runtime()
    if rt is None:
        pytest.skip("no clang ASan runtime next to hipcc")
    return build_asan, rt


def _env(rt, lib):
    return dict(os.environ, LD_PRELOAD=rt, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:exitcode=23",
                MOE_LIB=lib)


def test_abi_host_tests_under_asan(asan):
    build_asan, rt = asan
    lib = build_asan.build()
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi_host.py")],
                       env=_env(rt, lib), cwd=ROOT, capture_output=True, text=True, timeout=900)
    out = r.stdout + r.stderr
    assert r.returncode == 0 and "AddressSanitizer" not in out, out[-4000:]
    assert " passed" in out


def test_asan_reports_a_planted_overflow(asan, tmp_path):
    """Negative control: a host function reading past a heap array, compiled and loaded as the
    library is, is caught."""
    build_asan, rt = asan
    from dropless_mixture_experts_device_amd.build import HIPCC
    src = tmp_path / "probe.hip"
    src.write_text(textwrap.dedent("""
        #include <hip/hip_runtime.h>
        extern "C" int probe_read_past_end(int n) {
            int* a = new int[n];
            for (int i = 0; i < n; ++i) a[i] = i;
            volatile int v = a[n];
            delete[] a;
            return v;
        }
    """))
    so = tmp_path / "libprobe.so"
    r = subprocess.run([HIPCC, "-shared", "-fPIC", "--offload-arch=gfx950", *build_asan.ASAN_COMPILE,
                        *build_asan.ASAN_LINK, str(src), "-o", str(so)], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    code = f"import ctypes; ctypes.CDLL({str(so)!r}).probe_read_past_end(4)"
    r = subprocess.run([sys.executable, "-c", code], env=_env(rt, ""), capture_output=True, text=True, timeout=120)
    assert r.returncode == 23 and "heap-buffer-overflow" in r.stderr, r.stderr[-2000:]
