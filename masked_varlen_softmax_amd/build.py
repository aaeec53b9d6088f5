"""Build libmvs.so in-tree for gfx950.

Host-only C++ (the range-table builder, diagnostics, error buffer) is compiled
with g++; the HIP sources with hipcc for gfx950 only. Packed fp32 vector
instructions are disabled on the device (``-packed-fp32-ops``). Objects go to
``_objs/`` beside this file, the library to ``libmvs.so``.
"""

from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OBJS = os.path.join(HERE, "_objs")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
HIPCC = os.path.join(ROCM, "bin", "hipcc")
ARCH = "gfx950"

HIP_SOURCES = ["prefill_bf16.hip", "prefill_f32.hip", "decode.hip", "table_device.hip", "api.hip"]
HOST_SOURCES = ["host.cpp"]

HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", f"-I{INCLUDE}", f"-I{CSRC}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fvisibility=hidden", "-Wall", "-Wno-unused-function",
]
HOST_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-fvisibility=hidden", f"-I{INCLUDE}", f"-I{CSRC}", "-Wall", "-Wextra"]


def library_path() -> str:
    return os.path.join(HERE, "libmvs.so")


# The sources that decide what a measured kernel does: its own file, the
# shared headers, and the entry points that size its launch.
KERNEL_SOURCES = {
    "prefill": ["api.hip", "common.hpp", "kernels.hpp", "mask.hpp", "prefill_bf16.hip"],
    "decode": ["api.hip", "common.hpp", "decode.hip", "kernels.hpp", "mask.hpp"],
}


def source_digest(kind: str | None = None) -> str:
    """sha256 over library sources (names and contents), to tie profiles to the code they measured.

    ``kind`` ("prefill" or "decode") restricts it to that kernel's sources; None covers every file.
    """
    import hashlib

    h = hashlib.sha256()
    names = sorted(os.listdir(CSRC)) if kind is None else KERNEL_SOURCES[kind]
    for name in names:
        h.update(name.encode())
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(ln for ln in (r.stderr or "").splitlines() if noise not in ln)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{err}")
    return err


def build_library(verbose: bool = False, extra_hip_flags=()) -> str:
    """Compile every source and link libmvs.so; returns the library path."""
    os.makedirs(OBJS, exist_ok=True)
    jobs = []
    for src in HIP_SOURCES:
        obj = os.path.join(OBJS, src + ".o")
        jobs.append([HIPCC, *HIP_FLAGS, *extra_hip_flags, "-c", os.path.join(CSRC, src), "-o", obj])
    for src in HOST_SOURCES:
        obj = os.path.join(OBJS, src + ".o")
        jobs.append(["g++", *HOST_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
    with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        for msg in ex.map(_run, jobs):
            if verbose and msg.strip():
                print(msg, file=sys.stderr)
    objs = [os.path.join(OBJS, s + ".o") for s in HIP_SOURCES + HOST_SOURCES]
    tmp = library_path() + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs])
    os.replace(tmp, library_path())
    return library_path()


if __name__ == "__main__":
    print(build_library(verbose=True))
