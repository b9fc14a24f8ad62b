"""Host code under AddressSanitizer, UndefinedBehaviorSanitizer and ThreadSanitizer.

Two drivers in tests/sanitize/, each built here with the sanitizers and run as a
child process:

  * oracle_driver.c calls every function of the C oracle (forward, row subset,
    blocked reference, probabilities, gradients with several threads, bias, key/value
    cache) on small inputs, plus its argument rejections -- under ASan + UBSan, and
    under TSan for the threaded paths;
  * abi_driver.c calls the C ABI's host code -- validation, launch planning, empty
    calls, status strings -- built with host-only sanitizer flags and linked with
    the kernel objects of the normal build.  None of its calls reaches a HIP call, so
    no GPU is involved.

A sanitizer report makes the child exit nonzero (-fno-sanitize-recover, halt_on_error).
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
ORACLE = [os.path.join(ROOT, "oracle", f) for f in
          ("attention_oracle.c", "attention_grad_oracle.c", "blocked_reference.c")]
CSRC = os.path.join(ROOT, "io_aware_attention_amd", "csrc")
BUILD = os.path.join(ROOT, "_build")
ROCM = "/opt/rocm"
ENV = dict(os.environ,
           ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
           UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1",
           TSAN_OPTIONS="halt_on_error=1")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    out = r.stdout + r.stderr
    assert r.returncode == 0, f"{' '.join(cmd)} -> {r.returncode}\n{out[-4000:]}"
    return out


def _check_clean(out: str, banner: str):
    assert banner in out, out[-4000:]
    for word in ("ERROR: AddressSanitizer", "runtime error:", "WARNING: ThreadSanitizer",
                 "ERROR: LeakSanitizer"):
        assert word not in out, out[-4000:]


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not installed")
@pytest.mark.parametrize("san", ["address,undefined", "thread"])
def test_oracle_under_sanitizer(tmp_path, san):
    exe = str(tmp_path / "oracle_driver")
    _run(["gcc", "-O1", "-g", "-std=gnu11", f"-fsanitize={san}", "-fno-sanitize-recover=all",
          "-fno-omit-frame-pointer", "-pthread", os.path.join(SAN, "oracle_driver.c"), *ORACLE,
          "-o", exe, "-lm"])
    _check_clean(_run([exe], env=ENV, timeout=300), "oracle driver: all calls clean")


def _kernel_objects():
    if not os.path.isdir(BUILD):
        return []
    return sorted(os.path.join(BUILD, f) for f in os.listdir(BUILD) if f.endswith(".hip.o"))


@pytest.mark.skipif(not os.path.exists(f"{ROCM}/bin/hipcc"), reason="hipcc not installed")
def test_abi_host_code_under_asan_ubsan(tmp_path):
    objs = _kernel_objects()
    if not objs:
        pytest.skip("kernel objects not built (run the package build first)")
    host = str(tmp_path / "fa355_san.o")
    drv = str(tmp_path / "abi_driver.o")
    exe = str(tmp_path / "abi_driver")
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all"]
    _run([f"{ROCM}/bin/hipcc", "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-x", "hip", *san,
          "-c", os.path.join(CSRC, "fa355.cpp"), "-o", host])
    _run([f"{ROCM}/llvm/bin/clang", "-O1", "-g", "-std=gnu11", "-D__HIP_PLATFORM_AMD__",
          "-I", f"{ROCM}/include", "-I", os.path.join(ROOT, "include"),
          "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
          "-c", os.path.join(SAN, "abi_driver.c"), "-o", drv])
    _run([f"{ROCM}/bin/hipcc", "--offload-arch=gfx950", *san, drv, host, *objs, "-o", exe])
    _check_clean(_run([exe], env=ENV, timeout=120), "abi driver: all calls clean")
