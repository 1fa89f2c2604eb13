"""Ahead-of-time build of the gfx950 library libsdm_amd.so (hipcc, no JIT).

`python -m sparse_delta_memory_amd.build` compiles every source under csrc/ into one shared
library next to this file. Device code is built for gfx950 only, with FP contraction off (only
explicit fmaf calls fuse) and the packed-FP32 instructions disabled.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libsdm_amd.so")
SOURCES = ["api.cpp", "phase1.hip", "phase1_tiled.hip", "dw.hip", "read.hip", "gds.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-ffp-contract=off", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def command(out: str = LIB) -> list[str]:
    """One hipcc call that compiles and links every source (for reference and the CPU tests)."""
    return [hipcc()] + FLAGS + ["-shared", "-I", INCLUDE, "-I", CSRC, "-o", out] + [os.path.join(CSRC, s) for s in SOURCES]


# Host-only sanitizers (AddressSanitizer, and UndefinedBehaviorSanitizer with traps, so no runtime
# beyond the ASan one is needed): each flag goes to the host compilation only, never to the gfx950
# device code.
SAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fsanitize-trap=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]
SAN_LIB = os.path.join(HERE, "libsdm_amd_san.so")


def build(verbose: bool = False, sanitize: bool = False) -> str:
    """Compile the library (always; the caller decides when): each source to an object file in
    parallel under a private build folder, then one link. Returns its path. sanitize: the host code
    built with ASan and UBSan into libsdm_amd_san.so instead (CPU checks of the host side; the
    process must preload the ASan runtime, see sanitize.py)."""
    flags = FLAGS + (SAN_FLAGS if sanitize else [])
    out_lib = SAN_LIB if sanitize else LIB
    import tempfile
    from concurrent.futures import ThreadPoolExecutor

    work = tempfile.mkdtemp(prefix="sdm_build_")
    try:
        def compile_one(src):
            obj = os.path.join(work, src + ".o")
            cmd = [hipcc()] + flags + ["-c", "-I", INCLUDE, "-I", CSRC, "-o", obj, os.path.join(CSRC, src)]
            if verbose:
                print(" ".join(cmd), flush=True)
            res = subprocess.run(cmd, capture_output=True, text=True)
            if res.returncode != 0:
                sys.stderr.write(res.stdout + res.stderr)
                raise RuntimeError("hipcc failed compiling %s" % src)
            return obj

        jobs = max(1, min(len(SOURCES), int(os.environ.get("MAX_JOBS", "0") or 0) or (os.cpu_count() or 1)))
        with ThreadPoolExecutor(max_workers=jobs) as ex:
            objs = list(ex.map(compile_one, SOURCES))
        tmp = out_lib + ".tmp%d" % os.getpid()
        cmd = [hipcc()] + flags + ["-shared", "-o", tmp] + objs
        if verbose:
            print(" ".join(cmd), flush=True)
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            sys.stderr.write(res.stdout + res.stderr)
            raise RuntimeError("hipcc failed linking %s" % out_lib)
        os.replace(tmp, out_lib)
    finally:
        shutil.rmtree(work, ignore_errors=True)
    return out_lib


if __name__ == "__main__":
    print(build(verbose=True))
