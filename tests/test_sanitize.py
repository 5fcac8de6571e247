"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

api.cpp (argument checks, workspace layouts, the T5 threshold construction)
is compiled with both sanitizers on its host side only, linked with
tests/abi_sanitize_driver.cpp and the library's kernel objects, and run on
the CPU: every check, size computation and refusal path of
include/fat5attn.h, and the thresholds of a sweep of T5 geometries, with
leak detection on.  No GPU is used (every call in the driver returns before
its first HIP call)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "attention_t5_relative_amd")
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
ROCM = "/opt/rocm"
KERNEL_OBJS = ["fwd.hip.o", "bwd.hip.o", "misc.hip.o", "norm_loss.hip.o", "fire.hip.o"]


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout[-4000:]}\n{r.stderr[-4000:]}"
    return r


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    hipcc = os.path.join(ROCM, "bin", "hipcc")
    clang = os.path.join(ROCM, "llvm", "bin", "clang++")
    if not (os.path.exists(hipcc) and os.path.exists(clang)):
        pytest.skip("ROCm compilers not installed")
    if not all(os.path.exists(os.path.join(BUILD, o)) for o in KERNEL_OBJS):
        from attention_t5_relative_amd import build
        build.build(jobs=min(8, os.cpu_count() or 1))
    d = tmp_path_factory.mktemp("sanitize")
    api = str(d / "api_san.o")
    # sanitizers on the host side of api.cpp only (its device side is one
    # static array)
    _run([hipcc, "-x", "hip", "-c", os.path.join(CSRC, "api.cpp"), "-o", api, "-fPIC",
          "-std=c++17", "--offload-arch=gfx950", "-I", os.path.join(ROOT, "include"), "-I", CSRC,
          "-O1", "-g", "-fno-omit-frame-pointer", "-Xclang", "-target-feature", "-Xclang",
          "-packed-fp32-ops",
          "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
          "-Xarch_host", "-fno-sanitize-recover=undefined"])
    drv = str(d / "driver.o")
    san = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined"]
    _run([clang, "-c", os.path.join(ROOT, "tests", "abi_sanitize_driver.cpp"), "-o", drv,
          "-std=c++17", "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROCM, "include"),
          "-D__HIP_PLATFORM_AMD__", "-O1", "-g", "-fno-omit-frame-pointer"] + san)
    exe = str(d / "abi_sanitize")
    _run([clang, "-o", exe, drv, api] + [os.path.join(BUILD, o) for o in KERNEL_OBJS]
         + san + ["-L" + os.path.join(ROCM, "lib"), "-lamdhip64",
                  "-Wl,-rpath," + os.path.join(ROCM, "lib")])
    yield exe
    shutil.rmtree(d, ignore_errors=True)


def test_abi_host_code_is_clean_under_asan_and_ubsan(driver):
    env = dict(os.environ,
               ASAN_OPTIONS="detect_leaks=1:abort_on_error=1:strict_string_checks=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([driver], capture_output=True, text=True, env=env, timeout=600)
    assert r.returncode == 0, r.stdout[-4000:] + r.stderr[-4000:]
    assert "Sanitizer" not in r.stderr, r.stderr[-4000:]
    assert "all expectations hold" in r.stdout
