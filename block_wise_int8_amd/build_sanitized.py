"""Host-side sanitizer build of the library and the oracle, for running the
CPU test suite under AddressSanitizer and UndefinedBehaviorSanitizer:

    python -m block_wise_int8_amd.build_sanitized
    LD_PRELOAD=$(gcc -print-file-name=libasan.so) ASAN_OPTIONS=detect_leaks=0 \\
        python -m pytest tests -m "not gpu" -p no:cacheprovider
    python -c "import __graft_entry__ as g; g.build()"   # the normal build again

What is sanitized is the host code the CPU suite runs: the C ABI layer
(abi.cpp: argument checks, error reporting, the tensor-parallel check), built
with g++, and the oracle (oracle.c), built with gcc.  The HIP sources are
compiled as in the normal build (device code cannot be sanitized; the CPU
suite never launches a kernel).  Both libraries are written to their usual
in-tree paths, replacing the normal builds until those are rebuilt.
"""
from __future__ import annotations

import os
import subprocess
import sys

from . import build as _b

SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g"]


def build() -> str:
    os.makedirs(_b.BUILD_DIR, exist_ok=True)
    objs = []
    for src in _b.SOURCES:
        obj = os.path.join(_b.BUILD_DIR, "san_" + os.path.splitext(src)[0] + ".o")
        objs.append(obj)
        path = os.path.join(_b.CSRC, src)
        if src.endswith(".hip"):
            cmd = [_b.hipcc()] + _b.compile_flags() + ["-x", "hip", "-c", path, "-o", obj]
        else:
            cmd = (["g++", "-std=c++17", "-O1", "-fPIC", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
                    "-I" + os.path.join(_b.ROOT, "include"), "-I" + _b.CSRC] + SAN + ["-c", path, "-o", obj])
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode:
            sys.stderr.write(r.stdout + r.stderr)
            raise RuntimeError("compile failed: " + src)
    tmp = _b.LIB_PATH + ".tmp%d" % os.getpid()
    subprocess.run(["g++", "-shared", "-fPIC"] + SAN + ["-o", tmp] + objs +
                   ["-L/opt/rocm/lib", "-Wl,-rpath,/opt/rocm/lib", "-lamdhip64"], check=True)
    _b.check_symbols(tmp)
    os.replace(tmp, _b.LIB_PATH)
    sys.path.insert(0, _b.ROOT)
    import oracle
    oracle.build(sanitize=True)
    return _b.LIB_PATH


if __name__ == "__main__":
    print(build())
