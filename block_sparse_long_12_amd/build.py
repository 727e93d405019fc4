"""Build libqsa.so for gfx950 with hipcc (in-tree, next to this file).

    python -m block_sparse_long_12_amd.build

Each HIP source is compiled to an object under _build/ (in parallel), then
hipcc links them into block_sparse_long_12_amd/libqsa.so.  No GPU is needed:
hipcc cross-compiles for gfx950.
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
BUILD_DIR = os.path.join(ROOT, "_build", "libqsa")
LIB_PATH = os.path.join(HERE, "libqsa.so")

SOURCES = ["rope.hip", "compress.hip", "index_scores.hip", "select.hip", "prefill_select.hip",
           "attention.hip", "decode.hip", "paged.hip", "gdn.hip", "qsa_abi.hip"]
ARCH = os.environ.get("QSA_OFFLOAD_ARCH", "gfx950")

FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # packed fp32 ops stay off: hipcc -O3 would otherwise form v_pk_* FP32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fno-gpu-flush-denormals-to-zero",
    "-Wall", "-Wno-unused-function",
    f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}",
]


def _hipcc() -> str:
    for c in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def _run(cmd: list[str]) -> None:
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    if out.strip():
        print(out, file=sys.stderr)


def build(verbose: bool = False, jobs: int | None = None) -> str:
    """Compile every source and link libqsa.so; returns the library path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    hipcc = _hipcc()
    objs = []
    cmds = []
    for src in SOURCES:
        obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
        objs.append(obj)
        cmds.append([hipcc, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
    jobs = jobs or min(len(cmds), max(1, (os.cpu_count() or 2)))
    with ThreadPoolExecutor(jobs) as ex:
        for cmd, fut in zip(cmds, [ex.submit(_run, c) for c in cmds]):
            if verbose:
                print(" ".join(cmd))
            fut.result()
    tmp = LIB_PATH + ".tmp"
    _run([hipcc, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp, *objs])
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
