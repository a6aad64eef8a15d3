"""Builds libkvs.so in-tree for gfx950 with hipcc (one object per source,
compiled in parallel, then linked).  Usage: python -m non_uniform_sparse_amd.build"""

from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libkvs.so")
# Instrumented variant: decode workgroups record start/end stamps (skew runs only).
LIB_STAMPS = os.path.join(PKG, "libkvs_stamps.so")
# Measurement variant: the decode's logits on the VALU instead of MFMA (the
# comparison behind the MFMA choice; bench.py --logits valu).
LIB_VALU = os.path.join(PKG, "libkvs_valu.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

COMMON = ["-O3", "-fPIC", "-std=c++20", "-Wall", "-Wno-unused-function"]
# gfx950 device code; packed-fp32 instructions are switched off.
DEVICE = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-munsafe-fp-atomics"]


def sources(csrc: str = CSRC):
    return sorted(f for f in os.listdir(csrc) if f.endswith((".hip", ".cpp")))


def _compile(src: str, csrc: str = CSRC, build_dir: str = BUILD, defines=()) -> str:
    obj = os.path.join(build_dir, src + ".o")
    path = os.path.join(csrc, src)
    flags = [f"-I{os.path.join(ROOT, 'include')}", f"-I{csrc}", *COMMON, *defines]
    if src.endswith(".hip"):
        cmd = [HIPCC, "-x", "hip", *DEVICE, *flags, "-c", path, "-o", obj]
    else:  # host-only C++
        cmd = [HIPCC, *flags, "-c", path, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False, csrc: str = CSRC, lib: str = LIB,
          build_dir: str = BUILD, defines=()) -> str:
    """Compile every source under ``csrc`` and link ``lib``."""
    os.makedirs(build_dir, exist_ok=True)
    srcs = sources(csrc)
    with ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda f: _compile(f, csrc, build_dir, defines), srcs))
    tmp = lib + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-pthread", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)
    if verbose:
        print(f"built {lib}")
    return lib


def build_all(verbose: bool = False) -> None:
    """The library, its workgroup-stamp instrumented variant and its
    VALU-logits measurement variant."""
    build(verbose)
    build(verbose, lib=LIB_STAMPS, build_dir=BUILD + "_stamps", defines=("-DKVS_WG_STAMPS",))
    build(verbose, lib=LIB_VALU, build_dir=BUILD + "_valu", defines=("-DKVS_VALU_LOGITS",))


if __name__ == "__main__":
    build_all(verbose=True)
    sys.exit(0)
