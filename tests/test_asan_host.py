"""The C ABI's host code under AddressSanitizer, on the CPU: api.hip and
plan.cpp built with ASan on their host side (the device side is not
instrumented) and linked with launch functions that abort
(tests/asan_stubs.cpp), then tests/test_abi.py run against that library in
a child process with the ASan runtime preloaded. Every call there breaks an
argument rule or has no work, so none reaches a launch; an invalid memory
access in the checks, the plans or the status strings ends the run with an
AddressSanitizer report."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "attention_gqa_online_amd", "csrc")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
HIPCC = os.path.join(ROCM, "bin", "hipcc")
# ASan on the host pass only (each -fsanitize= right after -Xarch_host)
HOST_ASAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer"]


def _asan_runtime():
    clang = os.path.join(ROCM, "llvm", "bin", "clang")
    if not os.path.exists(clang):
        return None
    out = subprocess.run([clang, "-print-file-name=libclang_rt.asan-x86_64.so"],
                         capture_output=True, text=True).stdout.strip()
    return out if os.path.isabs(out) and os.path.exists(out) else None


def test_host_checks_under_address_sanitizer(tmp_path):
    rt = _asan_runtime()
    if not os.path.exists(HIPCC) or rt is None:
        pytest.skip("hipcc or the ASan runtime is not available")
    so = str(tmp_path / "libattn_asan.so")
    subprocess.run([HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-shared",
                    *HOST_ASAN, "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                    "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-o", so,
                    os.path.join(CSRC, "api.hip"), os.path.join(CSRC, "plan.cpp"),
                    os.path.join(ROOT, "tests", "asan_stubs.cpp")],
                   check=True, capture_output=True, text=True)
    if shutil.which("nm"):  # the host code really is instrumented
        undef = subprocess.run(["nm", "-D", "--undefined-only", so], capture_output=True,
                               text=True, check=True).stdout
        assert "__asan_" in undef
    env = dict(os.environ, LD_PRELOAD=rt, ATTN_GQA_LIB=so,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:halt_on_error=1")
    proc = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                           os.path.join(ROOT, "tests", "test_abi.py")],
                          cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = proc.stdout + proc.stderr
    assert "AddressSanitizer" not in out, out[-4000:]
    assert proc.returncode == 0, out[-4000:]
    assert " passed" in proc.stdout
