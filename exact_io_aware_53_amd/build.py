"""Build libfa.so (HIP kernels + C ABI) for gfx950 with hipcc, in-tree.

    python -m exact_io_aware_53_amd.build        # or build() from Python

Every source under csrc/ is compiled to an object in parallel, then linked
into exact_io_aware_53_amd/libfa.so. The build always recompiles.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libfa.so")
ARCH = "gfx950"

# Packed-fp32 VALU forms are kept out of the generated code. Matrix-core
# results are kept in architectural VGPRs, so the softmax can work on them
# without copies out of the accumulation registers.
COMMON = ["-O3", "-fPIC", "-std=c++17", f"--offload-arch={ARCH}",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-mllvm", "-amdgpu-mfma-vgpr-form=1",
          "-Wno-unused-command-line-argument"]


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP toolchain is required to build libfa.so")


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC)
                  if f.endswith(".hip") or f.endswith(".cpp"))


def flags(src: str):
    """Compile flags of one source. Kernels of head size 256 (*_d256.hip) hold
    more than 256 registers per lane, so they let matrix-core accumulators live
    in the AGPR half of the register file."""
    if src.endswith("_d256.hip"):
        return [f for f in COMMON if f not in ("-mllvm", "-amdgpu-mfma-vgpr-form=1")]
    return COMMON


def _compile(src: str, defines=(), build_dir=BUILD) -> str:
    obj = os.path.join(build_dir, os.path.basename(src) + ".o")
    cmd = [hipcc(), "-x", "hip", *flags(src), *[f"-D{d}" for d in defines], "-c", src, "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    return obj


def build(verbose: bool = False, defines=(), lib_path: str = LIB, build_dir: str = BUILD) -> str:
    """Compile every source (optionally with extra -D defines) and link `lib_path`."""
    os.makedirs(build_dir, exist_ok=True)
    srcs = sources()
    workers = max(1, min(len(srcs), os.cpu_count() or 1, 8))
    with ThreadPoolExecutor(max_workers=workers) as ex:
        objs = list(ex.map(lambda s: _compile(s, defines, build_dir), srcs))
    tmp = lib_path + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, lib_path)
    if verbose:
        print(f"built {lib_path} from {len(srcs)} sources")
    return lib_path


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
