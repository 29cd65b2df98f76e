"""Build liblora.so (the HIP library behind include/lora.h) for gfx950.

``python -m bwd_adamw_amd.build`` compiles in-tree with hipcc; the shared
object lands next to this file so that it travels with the source tree.  The
entry points and the GEMM instances of each quantized-W format are separate
translation units, compiled in parallel and linked into one library.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
SRCS = [os.path.join(CSRC, f) for f in
        ("lora_api.hip", "gemm_q8_0.hip", "gemm_q4_0.hip", "gemm_q4_k.hip", "gemm_q6_k.hip")]
OUT = os.path.join(HERE, "liblora.so")
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    # no packed-FP32 instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP toolchain is required to build liblora")


def _run(cmd, verbose):
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{' '.join(cmd)}\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)


def build(verbose: bool = False) -> str:
    """Compile liblora.so; always recompiles.  Returns the library path."""
    cc = hipcc()
    objs = [os.path.join(CSRC, os.path.basename(src) + ".o.tmp") for src in SRCS]
    jobs = max(1, min(len(SRCS), os.cpu_count() or 1, 16))
    try:
        with ThreadPoolExecutor(jobs) as pool:
            for f in [pool.submit(_run, [cc, *HIPCC_FLAGS, "-c", src, "-o", obj], verbose)
                      for src, obj in zip(SRCS, objs)]:
                f.result()
        tmp = OUT + ".tmp"
        _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
        os.replace(tmp, OUT)
    finally:
        for obj in objs:
            if os.path.exists(obj):
                os.remove(obj)
    return OUT


if __name__ == "__main__":
    print(build(verbose=True))
