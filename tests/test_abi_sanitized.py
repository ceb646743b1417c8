"""CPU: the C-ABI tests (tests/test_abi.py, tests/test_binding_checks.py) rerun
against libts_san.so -- api.cpp's host code built with AddressSanitizer and
UndefinedBehaviorSanitizer (no recovery) -- in a child process that preloads the
sanitizer runtime of the compiler that built it. Any report fails the run."""
import glob
import os
import subprocess
import sys

import pytest

from long_context_kv_ts_amd import build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _asan_runtime():
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    hits = sorted(glob.glob(os.path.join(rocm, "lib", "llvm", "lib", "clang", "*", "lib", "linux",
                                         "libclang_rt.asan-x86_64.so")))
    hits += sorted(glob.glob(os.path.join(rocm, "lib", "llvm", "lib", "clang", "*", "lib",
                                          "x86_64-unknown-linux-gnu", "libclang_rt.asan.so")))
    return hits[-1] if hits else None


def test_abi_checks_under_address_and_ub_sanitizers(tmp_path):
    rt = _asan_runtime()
    if rt is None:
        pytest.skip("no clang AddressSanitizer runtime under ROCM_PATH")
    if not os.path.exists(build.SAN_LIB):
        build.build_host_sanitized(verbose=False)
    env = dict(os.environ)
    env["TS_LIBRARY"] = build.SAN_LIB
    env["LD_PRELOAD"] = rt + (":" + env["LD_PRELOAD"] if env.get("LD_PRELOAD") else "")
    logs = str(tmp_path / "san")
    # the interpreter and torch are not instrumented: leak, ODR and allocator
    # pairing checks would report their allocations, not the library's
    env["ASAN_OPTIONS"] = f"detect_leaks=0:detect_odr_violation=0:alloc_dealloc_mismatch=0:log_path={logs}"
    env["UBSAN_OPTIONS"] = f"print_stacktrace=1:halt_on_error=1:log_path={logs}"
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu",
                        "tests/test_abi.py", "tests/test_binding_checks.py"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    reports = [open(f).read() for f in glob.glob(logs + "*")]
    assert not reports, "sanitizer report:\n" + "\n".join(reports)[:4000]
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert " passed" in r.stdout
