"""Build libqsa.so with AddressSanitizer and UndefinedBehaviorSanitizer on
its host code, then run pytest against that build.

    python -m block_sparse_long_12_amd.build_sanitize                 # the C-ABI tests (no GPU)
    python -m block_sparse_long_12_amd.build_sanitize -- <pytest args>

The sanitizers instrument the host pass only (each -fsanitize flag goes to
the host compiler): the argument checks of every entry point, the workspace
carving, the launch set-up and the per-device scratch bookkeeping.  Device
code is compiled as in build.py.  The library goes to
_build/sanitize/libqsa.so; pytest runs in a child process with the ASan
runtime preloaded ahead of anything already preloaded (the interpreter
itself is not instrumented) and
QSA_LIBRARY naming that library, so a sanitizer report fails the run.
Leak checking is off: the interpreter and torch keep allocations until exit.
"""

from __future__ import annotations

import glob
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

from block_sparse_long_12_amd import build as B

OUT_DIR = os.path.join(B.ROOT, "_build", "sanitize")
LIB_PATH = os.path.join(OUT_DIR, "libqsa.so")
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]


def asan_runtime() -> str:
    """The clang ASan runtime matching hipcc's compiler."""
    rocm = os.path.dirname(os.path.dirname(os.path.realpath(B._hipcc())))
    for root in (os.path.join(rocm, "llvm"), os.path.join(rocm, "lib", "llvm"), "/opt/rocm/llvm"):
        hits = sorted(glob.glob(os.path.join(root, "lib", "clang", "*", "lib", "linux", "libclang_rt.asan-x86_64.so")))
        if hits:
            return hits[-1]
    raise RuntimeError("libclang_rt.asan-x86_64.so not found next to hipcc")


def build() -> str:
    os.makedirs(OUT_DIR, exist_ok=True)
    hipcc = B._hipcc()
    flags = [f for f in B.FLAGS if f != "-O3"] + ["-O1", "-g"] + HOST_SAN
    cmds, objs = [], []
    for src in B.SOURCES:
        obj = os.path.join(OUT_DIR, os.path.splitext(src)[0] + ".o")
        objs.append(obj)
        cmds.append([hipcc, *flags, "-c", os.path.join(B.CSRC, src), "-o", obj])
    with ThreadPoolExecutor(min(len(cmds), os.cpu_count() or 2)) as ex:
        for f in [ex.submit(B._run, c) for c in cmds]:
            f.result()
    B._run([hipcc, "-shared", "-fPIC", f"--offload-arch={B.ARCH}", *HOST_SAN, "-shared-libsan", "-o", LIB_PATH,
            *objs])
    return LIB_PATH


def run_pytest(args: list[str]) -> int:
    env = dict(os.environ)
    env["QSA_LIBRARY"] = LIB_PATH
    pre = env.get("LD_PRELOAD", "")
    env["LD_PRELOAD"] = asan_runtime() + (":" + pre if pre else "")     # the runtime first, nothing removed
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    return subprocess.call([sys.executable, "-m", "pytest", *args], cwd=B.ROOT, env=env)


if __name__ == "__main__":
    argv = sys.argv[1:]
    pytest_args = argv[argv.index("--") + 1:] if "--" in argv else ["tests/test_abi_cpu.py", "-q"]
    print(build())
    sys.exit(run_pytest(pytest_args))
