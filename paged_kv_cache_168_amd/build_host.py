"""Build the host code alone (pa_host.cpp: argument checks and the host checkers of the device-data
preconditions; pa_engine.cpp: the block manager and scheduler) with a plain C++ compiler, by default under
AddressSanitizer and UndefinedBehaviorSanitizer. The result exports the same host functions as libpa.so; the
binding uses it in place of libpa.so for them when PA_HOST_LIBRARY names it (the sanitizer tier of the CPU
tests). Run as ``python -m paged_kv_cache_168_amd.build_host OUT``."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
HOST_SOURCES = ["pa_host.cpp", "pa_engine.cpp"]
SANITIZE = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer"]


def build_host(out: str, sanitize: bool = True) -> str:
    cxx = os.environ.get("CXX", "g++")
    srcs = [os.path.join(HERE, "csrc", s) for s in HOST_SOURCES]
    flags = ["-std=c++17", "-O1", "-g", "-shared", "-fPIC", "-Wall", "-Wextra", "-I", os.path.join(ROOT, "include")]
    cmd = [cxx] + flags + (SANITIZE if sanitize else []) + srcs + ["-o", out]
    subprocess.run(cmd, check=True)
    return out


if __name__ == "__main__":
    print(build_host(sys.argv[1] if len(sys.argv) > 1 else os.path.join(HERE, "libpa_host_san.so")))
