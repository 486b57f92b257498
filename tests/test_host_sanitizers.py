"""The C ABI's argument and shape checks (csrc/api.hip) built for the host with
AddressSanitizer and UndefinedBehaviorSanitizer, the kernel launchers replaced by the
stand-ins of tests/host_check/launch_stubs.hip, and test_abi.py's argument-check cases run
against that build in a child process.  A read or write out of bounds, a use of freed
memory, or undefined behaviour (a signed overflow in a size product, a misaligned access, a
bad shift) on any error path stops the child with the sanitizer's report.  Host code only:
the library's GPU code is not part of this build, and the check needs no GPU."""
import glob
import os
import shutil
import subprocess
import sys

import pytest

from conftest import ROOT, gpu_available

HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
ASAN_RT = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
# every sanitizer flag goes to the host pass only
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all"]
FLAGS = ["-O1", "-g", "-std=c++17", "-fPIC", "--offload-arch=gfx950", "--offload-host-only",
         "-fno-omit-frame-pointer", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", os.path.join(ROOT, "include")]
SOURCES = [os.path.join(ROOT, "block_sparse_top_ssa_amd", "csrc", "api.hip"),
           os.path.join(ROOT, "tests", "host_check", "launch_stubs.hip")]


def _run(cmd, **kw):
    p = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert p.returncode == 0, f"{' '.join(cmd)}\n{p.stdout[-4000:]}\n{p.stderr[-4000:]}"
    return p


@pytest.mark.skipif(not os.path.exists(HIPCC) or not ASAN_RT, reason="hipcc or the clang ASan runtime is missing")
@pytest.mark.skipif(gpu_available(), reason="the stand-in launchers are for a host without a GPU")
def test_argument_checks_under_asan_and_ubsan(tmp_path):
    objs = []
    for src in SOURCES:
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        _run([HIPCC, *FLAGS, *HOST_SAN, "-c", src, "-o", obj])
        objs.append(obj)
    lib = str(tmp_path / "libssa_hostcheck.so")
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *HOST_SAN, *objs, "-o", lib])
    # the build is instrumented: it calls into both runtimes
    undef = _run(["nm", "--undefined-only", lib]).stdout
    assert "__asan_report_" in undef and "__ubsan_handle_" in undef

    env = dict(os.environ, SSA_HOST_CHECK_LIB=lib, LD_PRELOAD=ASAN_RT[-1],
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:exitcode=86",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1:exitcode=87")
    p = subprocess.run([sys.executable, "-m", "pytest", "-q", "-s", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi.py"), "-k", "not exports and not probe"],
                       env=env, cwd=ROOT, capture_output=True, text=True, timeout=900)
    out = p.stdout[-6000:] + p.stderr[-6000:]
    assert p.returncode == 0, out
    assert "ERROR: AddressSanitizer" not in out and "runtime error" not in out, out
    assert " passed" in p.stdout and " failed" not in p.stdout, out
