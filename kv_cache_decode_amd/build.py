"""Build ``libkvdecode.so`` (the C-ABI HIP library) for gfx950 with hipcc.

Every HIP source is compiled with packed-fp32 instructions disabled: hipcc
would otherwise fuse pairs of fp32 operations into v_pk_* forms by itself.
The host pass prints that it does not know the feature; that is expected.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libkvdecode.so")
BUILD_DIR = os.path.join(HERE, "_build")
ARCH = os.environ.get("KVD_OFFLOAD_ARCH", "gfx950")

SOURCES = ["kvd_index.hip", "kvd_attn.hip", "kvd_quant.hip", "kvd_cache.hip", "kvd_probe.hip", "kvd_check.hip",
           "kvd_tier.hip", "kvd_api.hip"]
COMMON = ["-std=c++17", "-O3", "-fPIC", f"--offload-arch={ARCH}", "-Wall", "-Wno-unused-result",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: install ROCm or put /opt/rocm/bin on PATH")


def _compile(src: str, verbose: bool, build_dir: str, defines) -> str:
    obj = os.path.join(build_dir, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *COMMON, *[f"-D{d}" for d in defines], "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msgs = [l for l in (r.stdout + r.stderr).splitlines() if noise not in l]
    if msgs and (verbose or r.returncode):
        print("\n".join(msgs), file=sys.stderr)
    if r.returncode:
        raise RuntimeError(f"hipcc failed on {src}")
    return obj


def build(verbose: bool = False, out: str = LIB, defines=()) -> str:
    """Compile and link the library to ``out``; ``defines`` are extra -D macros
    (launch-shape knobs of the kernel sources)."""
    build_dir = BUILD_DIR if out == LIB else out + ".build"
    os.makedirs(build_dir, exist_ok=True)
    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose, build_dir, defines), SOURCES))
    tmp = out + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True, capture_output=not verbose)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
