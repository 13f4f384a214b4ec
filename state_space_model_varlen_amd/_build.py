"""Build the HIP library ``libssd_mi355x.so`` in-tree for gfx950 with hipcc."""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libssd_mi355x.so")
SOURCES = ["ssd_api.cpp", "ssd_prefill.hip", "ssd_decode.hip", "ssd_replay.hip",
           "ssd_noalloc.hip"]
HEADERS = ["ssd_device.h", "ssd_launch.h"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 instructions stay off (the compiler would otherwise form
    # v_pk_* from float2 code)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed building libssd_mi355x.so")


def build(verbose: bool = False) -> str:
    """Compile every source (in parallel, one hipcc per file) and link the shared
    library (always rebuilds)."""
    tag = f".tmp{os.getpid()}"
    inc = ["-I", os.path.join(PKG, "..", "include")]
    objs = [os.path.join(CSRC, s + tag + ".o") for s in SOURCES]
    jobs = [[hipcc()] + HIPCC_FLAGS + inc + ["-c", "-o", o, os.path.join(CSRC, s)]
            for s, o in zip(SOURCES, objs)]
    try:
        with ThreadPoolExecutor(max_workers=min(len(jobs), os.cpu_count() or 1, 8)) as ex:
            for f in [ex.submit(_run, j, verbose) for j in jobs]:
                f.result()
        tmp = LIB + tag
        _run([hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs, verbose)
        os.replace(tmp, LIB)
    finally:
        for o in objs:
            if os.path.exists(o):
                os.remove(o)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
