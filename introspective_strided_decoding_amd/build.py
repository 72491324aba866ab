"""Build libisd.so (HIP kernels for gfx950 + the C ABI) in-tree with hipcc.

    python introspective_strided_decoding_amd/build.py

(run as a script: importing the package loads the library this builds).

Every source is compiled to an object under _build/ and linked into
introspective_strided_decoding_amd/libisd.so.  Packed-fp32 VALU instructions
are disabled in device code.
"""

from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libisd.so")
ARCH = "gfx950"

SOURCES = ["isd_api.cpp", "attention.hip", "accept.hip", "commit.hip", "propose.hip", "loop.hip", "lora.hip", "gated_linear.hip"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found; the HIP toolchain is required to build libisd.so")


def _flags():
    return ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", INCLUDE, "-I", CSRC,
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wall", "-Wno-unused-function"]


def _compile(src: str, build_dir: str = BUILD, extra=()) -> str:
    obj = os.path.join(build_dir, os.path.basename(src) + ".o")
    cmd = [hipcc()] + _flags() + list(extra) + ["-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd.insert(1, "-xhip")
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{err}")
    if err.strip():
        sys.stderr.write(err + "\n")
    return obj


# Host code instrumented with AddressSanitizer and UndefinedBehaviorSanitizer
# (device code is built as usual): each -fsanitize= applies to the host pass only.
HOST_SANITIZERS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                   "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=all"]


def build(verbose: bool = False, out: str = LIB, extra=(), link_extra=()) -> str:
    """Compile every source and link ``out``; ``extra`` is added to every compile line and
    ``link_extra`` to the link line (HOST_SANITIZERS for the sanitizer build)."""
    build_dir = BUILD if out == LIB else os.path.join(BUILD, os.path.basename(os.path.dirname(out)) or "alt")
    os.makedirs(build_dir, exist_ok=True)
    srcs = list(SOURCES)
    missing = [s for s in srcs if not os.path.exists(os.path.join(CSRC, s))]
    if missing:
        raise RuntimeError(f"missing sources: {missing}")
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda src: _compile(src, build_dir, extra), srcs))
    tmp = out + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC"] + list(link_extra) + ["-o", tmp] + objs
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{res.stderr}")
    os.replace(tmp, out)
    if verbose:
        print(f"built {out}")
    return out


if __name__ == "__main__":
    build(verbose=True)
