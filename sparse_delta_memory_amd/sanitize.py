"""CPU run of the test suite under AddressSanitizer and UndefinedBehaviorSanitizer.

    python -m sparse_delta_memory_amd.sanitize [pytest args...]

Builds the host side of the library (the C ABI's checks, the launch planners) with ASan and UBSan
(libsdm_amd_san.so; the gfx950 device code is built as usual) and the C oracle the same way
(oracle/libsdm_oracle_san.so), then runs `pytest -m "not gpu"` in a child process that preloads
the ROCm clang ASan runtime and loads those two libraries (SDM_LIB, SDM_ORACLE_LIB). UB traps
(SIGILL) and ASan reports end the child with a non-zero status. Leak checking is off: the Python
interpreter itself is not built with the sanitizer and keeps allocations until exit.
"""

from __future__ import annotations

import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


def asan_runtime() -> str:
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not hits:
        raise RuntimeError("the ROCm clang ASan runtime (libclang_rt.asan-x86_64.so) was not found")
    return hits[-1]


def main(argv) -> int:
    sys.path.insert(0, ROOT)
    from sparse_delta_memory_amd import build as hipbuild
    import oracle

    lib = hipbuild.build(sanitize=True)
    olib = oracle.build(sanitize=True)
    env = dict(os.environ)
    env.update(SDM_LIB=lib, SDM_ORACLE_LIB=olib, LD_PRELOAD=asan_runtime(),
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:halt_on_error=1:verify_asan_link_order=0")
    cmd = [sys.executable, "-m", "pytest", os.path.join(ROOT, "tests"), "-q", "-m", "not gpu", "-p", "no:cacheprovider"] + list(argv)
    print(" ".join(cmd), flush=True)
    return subprocess.call(cmd, cwd=ROOT, env=env)


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))
