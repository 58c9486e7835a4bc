"""Build libcabf.so (HIP for gfx950) in-tree, and the benchmark's measurement
aid libcabf_probe.so (a dense matrix-core loop, not part of the library's ABI).

Every call recompiles every source: ``python content_adaptive_block_fractal_amd/build.py``
(run as a file: importing the package first would load the library it builds).
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
LIB = os.path.join(HERE, "libcabf.so")
PROBE_SRC = os.path.join(HERE, "probe", "mfma_peak.hip")
PROBE_LIB = os.path.join(HERE, "libcabf_probe.so")

SOURCES = ["api.cpp", "permute.hip", "mask.hip", "mask_noalloc.hip", "attention.hip",
           "attention_simple.hip", "attention_mfma.hip", "attention_pair.hip", "attention_bwd.hip", "kmeans.hip", "svg.hip",
           ]

ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-fvisibility=hidden",
    # keep the compiler from emitting packed-fp32 VALU instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    path = src if os.path.isabs(src) else os.path.join(CSRC, src)
    cmd = [_hipcc(), *FLAGS, "-x", "hip", "-c", path, "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"compiling {src} failed:\n{' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    noisy = [ln for ln in res.stderr.splitlines() if "packed-fp32-ops" not in ln and ln.strip()]
    if noisy:
        sys.stderr.write("\n".join(noisy) + "\n")
    return obj


def _link(objs, out: str):
    tmp = out + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"linking failed:\n{' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, out)


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    sources = [s for s in SOURCES if os.path.exists(os.path.join(CSRC, s))]
    jobs = min(len(sources) + 1, int(os.environ.get("MAX_JOBS", "8")))
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        probe = ex.submit(_compile, PROBE_SRC)
        objs = list(ex.map(_compile, sources))
        probe_obj = probe.result()
    _link(objs, LIB)
    _link([probe_obj], PROBE_LIB)
    if verbose:
        print(f"built {LIB} and {PROBE_LIB}")
    return LIB


if __name__ == "__main__":
    build()
