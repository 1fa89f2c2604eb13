"""The ctypes mirrors of the C structs in include/sdm.h have the C layout: every field at the same
offset, every struct the same size (CPU only: the header is compiled for the host with gcc and
prints offsetof / sizeof)."""

import ctypes
import os
import shutil
import subprocess
import tempfile

import pytest

from sparse_delta_memory_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIP_INCLUDE = "/opt/rocm/include"
STRUCTS = [("sdm_p1_shape", _lib.P1Shape), ("sdm_p1_io", _lib.P1IO), ("sdm_dw_io", _lib.DwIO),
           ("sdm_read_io", _lib.ReadIO), ("sdm_gds_io", _lib.GdsIO),
           ("sdm_gwr_io", _lib.GwrIO), ("sdm_pa_io", _lib.PaIO)]

pytestmark = pytest.mark.skipif(shutil.which("gcc") is None or
                                not os.path.exists(os.path.join(HIP_INCLUDE, "hip", "hip_runtime_api.h")),
                                reason="gcc or the HIP headers are missing")


def test_ctypes_mirrors_match_c_layout():
    lines = ["#include <stdio.h>", "#include <stddef.h>", '#include "sdm.h"', "int main(void) {"]
    for cname, cls in STRUCTS:
        lines.append('    printf("%s sizeof %%zu\\n", sizeof(%s));' % (cname, cname))
        for fname, _ in cls._fields_:
            lines.append('    printf("%s %s %%zu\\n", offsetof(%s, %s));' % (cname, fname, cname, fname))
    lines += ["    return 0;", "}"]
    with tempfile.TemporaryDirectory() as d:
        src, exe = os.path.join(d, "layout.c"), os.path.join(d, "layout")
        with open(src, "w") as f:
            f.write("\n".join(lines) + "\n")
        subprocess.run(["gcc", "-std=c11", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"),
                        "-I", HIP_INCLUDE, src, "-o", exe], check=True, capture_output=True)
        out = subprocess.run([exe], check=True, capture_output=True, text=True).stdout.split("\n")
    c = {}
    for line in out:
        if line:
            s, f, v = line.split()
            c[(s, f)] = int(v)
    for cname, cls in STRUCTS:
        assert c[(cname, "sizeof")] == ctypes.sizeof(cls), cname
        for fname, _ in cls._fields_:
            assert c[(cname, fname)] == getattr(cls, fname).offset, (cname, fname)
