"""Build ``libpa.so`` (gfx950) in-tree with hipcc.

Run as ``python -m paged_kv_cache_168_amd.build``. Compiles every HIP/C++
source under ``csrc/`` for gfx950 into one shared library next to this file.
"""
from __future__ import annotations

import os
import subprocess
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libpa.so")
SOURCES = ["pa_api.cpp", "pa_host.cpp", "pa_decode.hip", "pa_decode_balanced.hip", "pa_prefill.hip", "pa_cache.hip", "pa_engine.cpp", "pa_probe.hip"]
ARCH = os.environ.get("PA_OFFLOAD_ARCH", "gfx950")

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Wall",
    # packed FP32 instructions are kept out of every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA results and accumulators stay in ordinary VGPRs (no AGPR copies around the softmax)
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
    "-I", os.path.join(ROOT, "include"),
]


def build(verbose: bool = True, extra_flags=None, out: str = LIB) -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    # hipcc treats .cpp as host C++; force HIP language for every source so they share one code object
    cmd = [hipcc, "-x", "hip"] + srcs + HIPCC_FLAGS + list(extra_flags or []) + ["-o", out + ".tmp"]
    t0 = time.time()
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = [ln for ln in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in ln]
    if r.returncode != 0:
        sys.stderr.write("\n".join(msgs) + "\n")
        raise RuntimeError(f"hipcc failed ({r.returncode})")
    os.replace(out + ".tmp", out)
    if verbose:
        if msgs:
            print("\n".join(msgs))
        print(f"built {out} in {time.time() - t0:.1f}s")
    return out


if __name__ == "__main__":
    build()
