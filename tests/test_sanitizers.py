"""Address and undefined-behaviour sanitizer builds of the host code, run on the CPU.

* The oracle (``oracle/keops_oracle.c``) with gcc's ASan + UBSan (leak checking on),
  driven through every routine on small seeded inputs in exactly sized buffers
  (``tests/sanitize/oracle_driver.c``).
* The C ABI's host side (``geometric_map_reduce_amd/csrc/keops_api.cpp``: validation,
  block-sparse range checks, options) with the sanitizers on its host code only,
  linked with the library's other objects and driven by
  ``tests/sanitize/abi_host_driver.cpp``.  Every call there fails validation or
  reaches the first HIP call, which fails without a GPU; the driver refuses to run
  where a GPU is visible (its stand-in device addresses must never reach a kernel).
"""
from __future__ import annotations

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
CSRC = os.path.join(ROOT, "geometric_map_reduce_amd", "csrc")
OBJ = os.path.join(ROOT, "geometric_map_reduce_amd", "_build")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
CLANGXX = os.path.join(ROCM, "llvm", "bin", "clang++")
HIPCC = shutil.which("hipcc") or os.path.join(ROCM, "bin", "hipcc")


def _run(cmd, **kw):
    res = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert res.returncode == 0, f"{' '.join(cmd[:3])} ... failed ({res.returncode}):\n{res.stdout}\n{res.stderr}"
    return res


def test_oracle_under_asan_ubsan(tmp_path):
    if not shutil.which("gcc"):
        pytest.skip("gcc not available")
    exe = str(tmp_path / "oracle_driver")
    _run(["gcc", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
          "-fno-sanitize-recover=all", "-fopenmp", "-ffp-contract=off", "-std=c11",
          os.path.join(SAN, "oracle_driver.c"), os.path.join(ROOT, "oracle", "keops_oracle.c"), "-o", exe, "-lm"])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", OMP_NUM_THREADS="2",
               UBSAN_OPTIONS="print_stacktrace=1")
    res = _run([exe], env=env, timeout=300)
    assert "ok" in res.stdout and "runtime error" not in res.stderr


def test_abi_host_under_asan_ubsan(tmp_path):
    if os.path.exists("/dev/kfd"):
        pytest.skip("a GPU device node is present: this driver runs on hosts without a GPU only")
    if not (os.path.exists(CLANGXX) and os.path.exists(HIPCC)):
        pytest.skip("ROCm clang / hipcc not available")
    objs = sorted(os.path.join(OBJ, f) for f in os.listdir(OBJ) if f.endswith(".o") and f != "keops_api.cpp.o") \
        if os.path.isdir(OBJ) else []
    if not objs:
        pytest.skip("library objects not built")
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]
    api = str(tmp_path / "keops_api_san.o")
    drv = str(tmp_path / "driver.o")
    exe = str(tmp_path / "abi_host_driver")
    # sanitizers on the host code only (each -fsanitize= after -Xarch_host)
    _run([HIPCC, "-x", "hip", "--offload-arch=gfx950", "-fPIC", "-O1", "-g", "-fno-omit-frame-pointer",
          "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-std=c++17", *inc,
          "-c", os.path.join(CSRC, "keops_api.cpp"), "-o", api])
    _run([CLANGXX, "-O1", "-g", "-fno-omit-frame-pointer", "-fPIC", "-fsanitize=address,undefined",
          "-D__HIP_PLATFORM_AMD__", "-std=c++17", "-I", os.path.join(ROCM, "include"), *inc,
          "-c", os.path.join(SAN, "abi_host_driver.cpp"), "-o", drv])
    _run([CLANGXX, "-fsanitize=address,undefined", drv, api, *objs, "-L", os.path.join(ROCM, "lib"),
          "-Wl,-rpath," + os.path.join(ROCM, "lib"), "-lamdhip64", "-o", exe])
    # the HIP runtime keeps allocations until exit: leak checking off for this one
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0", UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    res = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    if res.returncode == 77:
        pytest.skip(res.stdout.strip())
    assert res.returncode == 0, f"driver failed ({res.returncode}):\n{res.stdout}\n{res.stderr[-4000:]}"
    assert "ok" in res.stdout and "runtime error" not in res.stderr
