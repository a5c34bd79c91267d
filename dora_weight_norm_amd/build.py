"""Build libdora.so in-tree with hipcc for gfx950.

    python -m dora_weight_norm_amd.build [-v]

Each HIP source compiles to an object under ``_build/`` (in parallel), then
they link into ``dora_weight_norm_amd/libdora.so``. The library links the HIP
runtime by its soname, so inside a process that has already imported torch
it binds to the runtime torch loaded.
"""

from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_PATH = os.path.join(HERE, "libdora.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = ["dora_api.hip", "norm_kernels.hip", "compose_kernels.hip"]

COMMON_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    # Correctly rounded fp32 sqrt and division; no implicit contraction.
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-ffp-contract=off",
    # No packed-fp32 instructions anywhere in the device code.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-I", os.path.join(ROOT, "include"),
]


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *COMMON_FLAGS, "-c", os.path.join(HERE, "csrc", src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(ln for ln in res.stderr.splitlines() if noise not in ln)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{err}")
    if err.strip() and verbose:
        print(err, file=sys.stderr)
    return obj


def build(verbose: bool = False) -> str:
    """Compile every HIP source for gfx950 and link libdora.so; returns its path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB_PATH + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stderr}")
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv[1:]))
