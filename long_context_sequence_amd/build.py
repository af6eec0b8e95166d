"""Builds libcp_attn.so in-tree with hipcc for gfx950 (no JIT cache, nothing installed).

Each source is compiled to an object in parallel, then linked into
long_context_sequence_amd/libcp_attn.so next to this file.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libcp_attn.so")
ARCH = os.environ.get("CP_ATTN_ARCH", "gfx950")

SOURCES = ["host.cpp", "host_fir.cpp", "fwd_bf16.hip", "fwd_f32.hip", "elementwise.hip",
           "bwd_bf16.hip", "fir.hip", "probe.hip", "noalloc.hip"]

# Packed fp32 instructions are kept out of the device code (-packed-fp32-ops).
HIP_FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Wall", "-Wno-unused-function", f"-I{INCLUDE}", f"-I{CSRC}"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libcp_attn.so)")


def _compile(src: str, verbose: bool, build_dir: str, defines) -> str:
    obj = os.path.join(build_dir, os.path.basename(src) + ".o")
    cmd = [hipcc(), *HIP_FLAGS, *[f"-D{d}" for d in defines], "-c", os.path.join(CSRC, src),
           "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(line for line in (res.stdout + res.stderr).splitlines()
                    if "packed-fp32-ops" not in line)
    if res.returncode != 0:
        raise RuntimeError(f"compiling {src} failed:\n{' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out, file=sys.stderr)
    return obj


def build(verbose: bool = False, out: str = LIB, defines=()) -> str:
    """Compile and link the library to `out` (default: the in-tree libcp_attn.so). `defines`
    override compile-time launch shapes (e.g. "CP_FWD_WAVES=8") for experiments."""
    build_dir = BUILD if out == LIB else out + ".objs"
    os.makedirs(build_dir, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose, build_dir, defines), SOURCES))
    tmp = out + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"linking failed:\n{' '.join(cmd)}\n{res.stdout}{res.stderr}")
    os.replace(tmp, out)
    return out


ABI_EXAMPLE_SRC = os.path.join(ROOT, "tests", "c_abi_ring.cpp")
ABI_EXAMPLE = os.path.join(BUILD, "c_abi_ring")


def build_abi_example(lib: str = LIB) -> str:
    """Compile the plain C++ consumer of the C ABI used by the tests (links the in-tree
    library with an rpath to it); output under _build/."""
    os.makedirs(BUILD, exist_ok=True)
    cmd = [hipcc(), "-O2", "-std=c++17", f"--offload-arch={ARCH}", f"-I{INCLUDE}", ABI_EXAMPLE_SRC,
           "-o", ABI_EXAMPLE, f"-L{os.path.dirname(lib)}", "-lcp_attn",
           f"-Wl,-rpath,{os.path.dirname(lib)}"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"compiling the ABI example failed:\n{' '.join(cmd)}\n{res.stdout}{res.stderr}")
    return ABI_EXAMPLE


if __name__ == "__main__":
    import argparse

    ap = argparse.ArgumentParser()
    ap.add_argument("--out", default=LIB)
    ap.add_argument("-D", dest="defines", action="append", default=[])
    a = ap.parse_args()
    print(build(verbose=True, out=os.path.abspath(a.out), defines=a.defines))
    if os.path.abspath(a.out) == LIB:
        print(build_abi_example())
