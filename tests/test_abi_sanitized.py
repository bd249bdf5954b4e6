"""The host side of the C ABI (argument checks, layouts, error strings)
under AddressSanitizer and UndefinedBehaviorSanitizer: the library is built
again with both sanitizers on its host code only (device code is untouched),
and the ABI tests run against that build in a child process with the ASan
runtime preloaded.  CPU only: every call the ABI tests make returns before
a kernel would launch."""
import glob
import os
import subprocess
import sys

import pytest

from fp4_compressed_sparse_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
RUNTIME = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))


@pytest.fixture(scope="module")
def sanitized_lib(tmp_path_factory):
    if not (os.path.exists(HIPCC) and RUNTIME):
        pytest.skip("hipcc or the clang ASan runtime is not installed")
    out = str(tmp_path_factory.mktemp("asan") / "libcsa2.so")
    san = []
    for f in ("address", "undefined"):                       # host code only
        san += ["-Xarch_host", "-fsanitize=" + f]
    flags = [f for f in B.FLAGS if f != "-O3"] + ["-O1", "-g", "-Xarch_host", "-fno-omit-frame-pointer",
                                                  "-Xarch_host", "-fno-sanitize-recover=undefined",
                                                  "-Xarch_host", "-shared-libasan"] + san
    r = subprocess.run([HIPCC] + flags + [os.path.join(ROOT, "fp4_compressed_sparse_amd", "csrc", "api.hip"),
                                          "-o", out], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    syms = subprocess.run(["nm", "-D", "--undefined-only", out], capture_output=True, text=True).stdout
    assert "__asan_" in syms and "__ubsan_" in syms      # the host code is instrumented
    return out


def test_abi_tests_clean_under_asan_ubsan(sanitized_lib):
    env = dict(os.environ)
    env.update(CSA2_LIB_PATH=sanitized_lib, LD_PRELOAD=RUNTIME[-1],
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    probe = ("import fp4_compressed_sparse_amd as c; c.load(); "
             "print(any('libclang_rt.asan' in l for l in open('/proc/self/maps')))")
    r = subprocess.run([sys.executable, "-c", probe], cwd=ROOT, env=env, capture_output=True, text=True)
    assert r.returncode == 0 and r.stdout.strip() == "True", r.stdout + r.stderr
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join("tests", "test_abi.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
