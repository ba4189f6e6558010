"""Build libks.so (HIP kernels + C ABI) for gfx950 with hipcc, in-tree.

    python -m kronecker_sparse_structured_amd.build [--incremental]

Every source in csrc/ is compiled to an object in parallel, then linked into
kronecker_sparse_structured_amd/lib/libks.so. The build always recompiles
everything, unless --incremental is given: then only sources whose object is
older than the source or any header are recompiled.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys
import time

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OBJ = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "lib", "libks.so")
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc"),
                 shutil.which("hipcc") or ""):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found; libks needs the ROCm toolchain")


COMMON = [
    "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-result",
    "--offload-arch=" + ARCH,
    # Keep the compiler from forming packed fp32 instructions on its own.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I" + INCLUDE, "-I" + CSRC,
]


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC)
                  if f.endswith(".hip") or f.endswith(".cpp"))


def _compile(src: str) -> str:
    obj = os.path.join(OBJ, os.path.basename(src) + ".o")
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = [hipcc(), *COMMON, *lang, "-c", src, "-o", obj]
    t0 = time.time()
    proc = subprocess.run(cmd, capture_output=True, text=True)
    if proc.returncode != 0:
        raise RuntimeError("compile failed: %s\n%s\n%s" % (" ".join(cmd), proc.stdout, proc.stderr))
    # The host pass does not know the packed-fp32 target feature and says so.
    noise = ("packed-fp32-ops", "not a recognized feature", "generated.")
    warn = "\n".join(l for l in proc.stderr.splitlines() if l.strip() and not any(n in l for n in noise))
    if warn:
        sys.stderr.write(warn + "\n")
    sys.stderr.write("  compiled %s in %.1fs\n" % (os.path.basename(src), time.time() - t0))
    return obj


def _stale(src: str) -> bool:
    """The object is missing or older than its source or any header."""
    obj = os.path.join(OBJ, os.path.basename(src) + ".o")
    if not os.path.exists(obj):
        return True
    headers = [os.path.join(d, f) for d in (CSRC, INCLUDE) for f in os.listdir(d) if f.endswith((".h", ".inc"))]
    newest = max(os.path.getmtime(p) for p in [src, *headers])
    return os.path.getmtime(obj) < newest


def build(jobs: int | None = None, incremental: bool = False) -> str:
    """Compile every source (or, with incremental=True, only those whose
    object is older than the source or a header) and link libks.so."""
    os.makedirs(OBJ, exist_ok=True)
    srcs = sources()
    todo = [s for s in srcs if _stale(s)] if incremental else srcs
    jobs = jobs or min(max(len(todo), 1), max(1, os.cpu_count() or 1), 16)
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        list(ex.map(_compile, todo))
    objs = [os.path.join(OBJ, os.path.basename(s) + ".o") for s in srcs]
    os.makedirs(os.path.dirname(LIB), exist_ok=True)
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc(), "--offload-arch=" + ARCH, "-shared", "-fPIC", *objs, "-o", tmp]
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    t0 = time.time()
    print(build(incremental="--incremental" in sys.argv[1:]))
    print("built in %.1fs" % (time.time() - t0))
