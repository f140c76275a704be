"""The host-side tests of the C ABI (tests/test_host_abi.py) again, in a child process
that loads the library's AddressSanitizer build (host code instrumented, device code
as usual) with the sanitizer runtime preloaded.  CPU only: nothing is launched."""

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, os.path.join(ROOT, "kv_cache_vector_fa_amd"))


def test_host_abi_under_address_sanitizer():
    import build
    lib = build.build_asan()
    rt = build.asan_runtime()
    assert os.path.exists(rt), rt
    env = dict(os.environ, LD_PRELOAD=rt, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               FA_TQ_LIB=lib)
    probe = ("import ctypes, kv_cache_vector_fa_amd as fa; l = fa.load(); "
             "assert fa.LIB_PATH.endswith('libfa_tq_asan.so'), fa.LIB_PATH; "
             "assert hasattr(ctypes.CDLL(None), '__asan_init'); print('asan build loaded')")
    r = subprocess.run([sys.executable, "-c", probe], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 0 and "asan build loaded" in r.stdout, r.stdout + r.stderr
    r = subprocess.run([sys.executable, "-m", "pytest", "tests/test_host_abi.py", "-q",
                        "-p", "no:cacheprovider", "-m", "not gpu"], cwd=ROOT, env=env,
                       capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert "passed" in r.stdout and "ERROR: AddressSanitizer" not in r.stderr
