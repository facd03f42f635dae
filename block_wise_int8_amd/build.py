"""Build ``libblockint8.so`` (HIP for gfx950) in-tree with hipcc.

    python -m block_wise_int8_amd.build

Every HIP source is compiled for gfx950 only, with:
  * ``-Xclang -target-feature -Xclang -packed-fp32-ops``: no packed-fp32 VALU
    forms are generated;
  * IEEE-correct fp32 division and kept denormals (the quantisation pass must
    be bit-exact);
  * ``-ffp-contract=off``: every fused multiply-add is written out explicitly.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD_DIR = os.path.join(PKG, "_build")
LIB_PATH = os.path.join(PKG, "libblockint8.so")
# the benchmark's shader-clock probe, a library of its own (not the product path)
CLOCK_LIB_PATH = os.path.join(PKG, "libbi8clock.so")

SOURCES = ["abi.cpp", "quant_act.hip", "gemm.hip", "moe.hip", "noalloc.hip"]
CLOCK_SOURCES = ["clockprobe.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm toolchain required to build libblockint8.so)")


def compile_flags() -> list[str]:
    return [
        "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-fno-gpu-flush-denormals-to-zero", "-fhip-fp32-correctly-rounded-divide-sqrt",
        "-ffp-contract=off", "-Wall", "-Wno-unused-function",
        "-I" + os.path.join(ROOT, "include"), "-I" + CSRC,
    ]


def _build_lib(sources: list[str], lib_path: str, verbose: bool, extra_flags: list[str] | None) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    cc = hipcc()
    flags = compile_flags() + list(extra_flags or [])
    procs = []
    objs = []
    for src in sources:
        obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
        objs.append(obj)
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        cmd = [cc] + flags + lang + ["-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
    failed = []
    for src, pr in procs:
        out, _ = pr.communicate()
        text = out.decode(errors="replace")
        # hipcc's host pass does not know the packed-fp32 feature; that note is harmless.
        text = "\n".join(l for l in text.splitlines() if "packed-fp32-ops" not in l)
        if text.strip() and (verbose or pr.returncode):
            print(text, file=sys.stderr)
        if pr.returncode:
            failed.append(src)
    if failed:
        raise RuntimeError("hipcc failed for: " + ", ".join(failed))
    tmp = lib_path + ".tmp%d" % os.getpid()
    link = [cc, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs
    if verbose:
        print(" ".join(link), flush=True)
    subprocess.run(link, check=True)
    check_symbols(tmp)
    os.replace(tmp, lib_path)
    return lib_path


def build(verbose: bool = False, extra_flags: list[str] | None = None) -> str:
    """Build libblockint8.so (and the benchmark's clock probe library)."""
    _build_lib(CLOCK_SOURCES, CLOCK_LIB_PATH, verbose, extra_flags)
    return _build_lib(SOURCES, LIB_PATH, verbose, extra_flags)


def check_symbols(path: str) -> None:
    """Fail the build if the library references a symbol of its own that no
    object defines (e.g. a kernel launch stub the host pass did not emit)."""
    nm = shutil.which("nm") or "/opt/rocm/llvm/bin/llvm-nm"
    out = subprocess.run([nm, "-u", path], check=True, capture_output=True, text=True).stdout
    missing = [l.split()[-1] for l in out.splitlines() if "bi8" in l or "blockint8" in l]
    if missing:
        raise RuntimeError("libblockint8.so has undefined internal symbols: " + ", ".join(missing))


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
