"""Build librkv.so (hand-written HIP for gfx950) in-tree with hipcc.

    python -m position_split_kv_amd.build        # or build() from Python

Every translation unit compiles in parallel; the split-kernel instances are
built once per K storage type.  Packed-FP32 instructions are disabled for the
device code (``-Xclang -target-feature -Xclang -packed-fp32-ops``).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "librkv.so")
# the streaming-read probe the benchmark measures the read ceiling with (not
# part of the attention library)
PROBE_LIB = os.path.join(HERE, "librkvprobe.so")
ARCH = os.environ.get("RKV_OFFLOAD_ARCH", "gfx950")

FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-result",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


def _hipcc() -> str:
    for c in ("/opt/rocm/bin/hipcc", shutil.which("hipcc") or ""):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def _units():
    units = []
    for kt in range(4):
        for vt in range(5):
            units.append((os.path.join(CSRC, "attend_inst.hip"), os.path.join(BUILD, f"attend_k{kt}_v{vt}.o"),
                          [f"-DRKV_KT={kt}", f"-DRKV_VT={vt}"]))
    for name in ("attend", "combine", "dequant", "append", "plan", "api"):
        units.append((os.path.join(CSRC, f"{name}.hip"), os.path.join(BUILD, f"{name}.o"), []))
    return units


def _compile(unit, incremental=False):
    src, obj, extra = unit
    if incremental and os.path.exists(obj):
        deps = [src] + [os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".h")]
        deps.append(os.path.join(ROOT, "include", "rkv.h"))
        if all(os.path.getmtime(d) <= os.path.getmtime(obj) for d in deps):
            return obj, ""
    cmd = [_hipcc(), *FLAGS, *extra, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj, r.stderr


def build(jobs: int | None = None, verbose: bool = False, incremental: bool = False) -> str:
    """Compile every HIP unit for gfx950 and link librkv.so.  By default every
    unit is rebuilt; ``incremental`` skips units whose object is newer than
    its sources (a development convenience)."""
    os.makedirs(BUILD, exist_ok=True)
    jobs = jobs or min(8, os.cpu_count() or 4)
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        results = list(ex.map(lambda u: _compile(u, incremental), _units()))
    if verbose:
        for obj, err in results:
            if err.strip():
                print(f"[{os.path.basename(obj)}]\n{err}", file=sys.stderr)
    tmp = LIB + ".tmp"
    cmd = [_hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp, *[o for o, _ in results]]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    tmp = PROBE_LIB + ".tmp"
    cmd = [_hipcc(), *FLAGS, "-shared", "-o", tmp, os.path.join(CSRC, "probe.hip")]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"probe build failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, PROBE_LIB)
    return LIB


if __name__ == "__main__":
    import time

    t = time.time()
    print(build(verbose="-v" in sys.argv, incremental="-i" in sys.argv), f"{time.time() - t:.1f}s")
