"""Build the AddressSanitizer check of the library's host-side validation layer.

Every csrc/*.hip file is compiled with AddressSanitizer on its host code only
(the device code is built as usual, but the driver never launches a kernel),
and linked with tests/asan/abi_driver.cpp into one executable.  CPU-only test
support; nothing here runs on a GPU.
"""
from __future__ import annotations

import concurrent.futures as cf
import hashlib
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
CSRC = os.path.join(ROOT, "input_adaptive_reduced_rmm_amd", "csrc")
INCLUDE = os.path.join(ROOT, "include")
OUT = os.path.join(HERE, "_build")

ASAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer"]
FLAGS = ["-O1", "-g", "-std=c++17", "--offload-arch=gfx950", "-Wall", "-Werror",
         "-Wno-unused-function", "-Wno-unused-parameter", "-Wno-unused-variable", "-Wno-unused-but-set-variable"]


def _sources():
    srcs = sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))
    deps = srcs + sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".h"))
    deps += [os.path.join(INCLUDE, "rmm.h"), os.path.join(HERE, "abi_driver.cpp"), os.path.abspath(__file__)]
    return srcs, deps


def build() -> str:
    """Compile (when the sources changed) and return the path of the ASan driver."""
    srcs, deps = _sources()
    h = hashlib.sha256()
    for p in deps:
        h.update(open(p, "rb").read())
    tag = h.hexdigest()[:16]
    exe = os.path.join(OUT, f"abi_driver_{tag}")
    if os.path.exists(exe):
        return exe
    os.makedirs(OUT, exist_ok=True)
    hipcc = "/opt/rocm/bin/hipcc"

    def compile_one(src):
        obj = os.path.join(OUT, os.path.basename(src) + ".o")
        cmd = [hipcc, *FLAGS, *ASAN, "-I", INCLUDE, "-I", CSRC, "-c", src, "-o", obj]
        if src.endswith(".cpp"):
            cmd = ["g++", "-O1", "-g", "-std=c++17", "-fsanitize=address", "-fno-omit-frame-pointer", "-Wall",
                   "-Werror", "-I", INCLUDE, "-c", src, "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"asan build failed on {src}:\n{r.stdout}{r.stderr}")
        return obj

    with cf.ThreadPoolExecutor(max_workers=8) as ex:
        objs = list(ex.map(compile_one, srcs + [os.path.join(HERE, "abi_driver.cpp")]))
    cmd = [hipcc, *ASAN, "--offload-arch=gfx950", "-o", exe + ".tmp", *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"asan link failed:\n{r.stdout}{r.stderr}")
    os.replace(exe + ".tmp", exe)
    return exe


if __name__ == "__main__":
    print(build())
    sys.exit(0)
