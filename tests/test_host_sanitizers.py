"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

wq_api.cpp (every argument check, the workspace bookkeeping, the error strings) is compiled with
host-side ASan and UBSan (the device code is built as usual), linked with the library's kernel
objects into a separate libwq.so, and tests/test_abi.py runs against it in a child process with
the clang ASan runtime preloaded. Any sanitizer report fails the test. No GPU is needed: every
call test_abi.py makes is refused on the host before a HIP call.
"""
import glob
import os
import subprocess
import sys

import pytest

import gemv_wq_gemm_amd.build as wq_build
from tests.conftest import ROOT

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CSRC = os.path.join(ROOT, "gemv_wq_gemm_amd", "csrc")
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=undefined"]


def _asan_runtime():
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


@pytest.fixture(scope="module")
def sanitized_lib(tmp_path_factory):
    if not os.access(HIPCC, os.X_OK) or _asan_runtime() is None:
        pytest.skip("hipcc or the clang ASan runtime is not available")
    b = wq_build
    out = tmp_path_factory.mktemp("asan")
    objs = []
    for src in [s for s in b.SOURCES if s.endswith(".hip")]:  # the kernels as the library builds them
        obj = os.path.join(b.OBJDIR, os.path.splitext(src)[0] + ".o")
        if not os.path.exists(obj) or os.path.getmtime(obj) < os.path.getmtime(os.path.join(CSRC, src)):
            os.makedirs(b.OBJDIR, exist_ok=True)
            b._compile(src)
        objs.append(obj)
    api = str(out / "wq_api.o")
    cmd = [HIPCC, "-x", "hip", "-O1", "-g", *[f for f in b.COMMON if f != "-O3"], *SAN,
           "-c", os.path.join(CSRC, "wq_api.cpp"), "-o", api]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    lib = str(out / "libwq.so")
    r = subprocess.run([HIPCC, f"--offload-arch={b.ARCH}", "-shared", "-fPIC", *SAN, api, *objs, "-o", lib],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return lib


def test_abi_checks_under_asan_and_ubsan(sanitized_lib):
    env = dict(os.environ)
    env.update(LD_PRELOAD=_asan_runtime(), ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", WQ_TEST_LIB=sanitized_lib)
    r = subprocess.run([sys.executable, "-m", "pytest", "tests/test_abi.py", "-q", "-p", "no:cacheprovider"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    report = r.stdout + r.stderr
    assert r.returncode == 0, report[-4000:]
    assert "AddressSanitizer" not in report and "runtime error" not in report, report[-4000:]
    assert " passed" in report
