"""Build the gfx950 shared library ``libkeops_mi355x.so`` from ``csrc/`` with hipcc.

Every translation unit is compiled for gfx950 only, with packed-fp32 code
generation disabled, in parallel, and linked in-tree next to this file:

    python -m geometric_map_reduce_amd.build          # or build() from Python
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OBJ = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libkeops_mi355x.so")
# instruction-rate microbenchmarks: a library of their own, never linked into LIB
MICRO_SRC = os.path.join(HERE, "micro", "rates.hip")
MICRO_LIB = os.path.join(HERE, "libkeops_micro.so")

HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17",
    # no packed fp32 (v_pk_*_f32) code generation anywhere
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA results in ordinary VGPRs: no accumulation-register copies before the
    # VALU reads them, and a smaller register footprint (more waves per SIMD)
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-Wall", "-Wno-unused-result", "-Wno-unused-value",
    "-I", INCLUDE, "-I", CSRC,
]


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp")))


def _compile(src: str) -> tuple[str, str]:
    obj = os.path.join(OBJ, os.path.basename(src) + ".o")
    cmd = [HIPCC, *CFLAGS, "-c", src, "-o", obj]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the device-only feature name; drop that note
    err = "\n".join(l for l in res.stderr.splitlines() if "not a recognized feature" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{err}")
    return obj, err


def _stale(src: str) -> bool:
    """True when the object of ``src`` is missing or older than the source or any header."""
    obj = os.path.join(OBJ, os.path.basename(src) + ".o")
    if not os.path.exists(obj):
        return True
    deps = [src] + [os.path.join(d, f) for d in (CSRC, INCLUDE) for f in os.listdir(d) if f.endswith(".h")]
    return os.path.getmtime(obj) < max(os.path.getmtime(p) for p in deps)


def build(jobs: int | None = None, verbose: bool = False, incremental: bool = False) -> str:
    """Compile every source (or, ``incremental``, those older than their inputs) and link
    the library; returns its path."""
    os.makedirs(OBJ, exist_ok=True)
    srcs = sources()
    todo = [s for s in srcs if _stale(s)] if incremental else srcs
    jobs = jobs or min(max(len(todo), 1), max(1, os.cpu_count() or 1), 16)
    with concurrent.futures.ThreadPoolExecutor(max_workers=jobs) as ex:
        results = list(ex.map(_compile, todo))
    if verbose:
        for _, err in results:
            if err.strip():
                print(err, file=sys.stderr)
    tmp = LIB + ".tmp%d" % os.getpid()
    objs = [os.path.join(OBJ, os.path.basename(s) + ".o") for s in srcs]
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stderr}")
    os.replace(tmp, LIB)
    build_micro()
    return LIB


def build_micro() -> str:
    """Compile the instruction-rate microbenchmarks into libkeops_micro.so (same flags)."""
    tmp = MICRO_LIB + ".tmp%d" % os.getpid()
    res = subprocess.run([HIPCC, *CFLAGS, "-shared", "-o", tmp, MICRO_SRC], capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {MICRO_SRC}:\n{res.stderr}")
    os.replace(tmp, MICRO_LIB)
    return MICRO_LIB


if __name__ == "__main__":
    print(build(verbose=True, incremental="--incremental" in sys.argv[1:]))
