"""Build libdora.so in-tree with hipcc for gfx950.

    python -m dora_weight_norm_amd.build [-v]

Each HIP source compiles to an object under ``_build/`` (in parallel), then
they link into ``dora_weight_norm_amd/libdora.so``. The library links the HIP
runtime by its soname, so inside a process that has already imported torch
it binds to the runtime torch loaded.
"""

from __future__ import annotations

import os
import re
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_PATH = os.path.join(HERE, "libdora.so")
# Per-kernel register, scratch and LDS use reported by the compiler (one line per kernel).
RESOURCE_REPORT = os.path.join(BUILD_DIR, "kernel_resources.txt")
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


def kernel_resources(remarks: str) -> dict:
    """{kernel: {field: value}} from hipcc's kernel-resource-usage remarks."""
    out, cur = {}, None
    for ln in remarks.splitlines():
        m = re.search(r"remark: (.*?) \[-Rpass-analysis=kernel-resource-usage\]", ln)
        if not m:
            continue
        text = m.group(1).strip()
        if text.startswith("Function Name:"):
            cur = text.split(":", 1)[1].strip()
            out[cur] = {}
        elif cur is not None and ":" in text:
            key, val = text.split(":", 1)
            out[cur][key.strip()] = val.strip()
    return out


def _compile(src: str, verbose: bool) -> tuple:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *COMMON_FLAGS, "-Rpass-analysis=kernel-resource-usage", "-c", os.path.join(HERE, "csrc", src),
           "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    lines = [ln for ln in res.stderr.splitlines() if noise not in ln]
    err = "\n".join(ln for ln in lines if "kernel-resource-usage" not in ln)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{err}")
    if err.strip() and verbose:
        print(err, file=sys.stderr)
    return obj, kernel_resources("\n".join(lines))


def build(verbose: bool = False) -> str:
    """Compile every HIP source for gfx950 and link libdora.so; returns its path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        done = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    objs = [o for o, _ in done]
    res_all = {}
    for _, r in done:
        res_all.update(r)
    with open(RESOURCE_REPORT, "w") as f:
        for name, d in sorted(res_all.items()):
            f.write(name + " " + " ".join(f"{k.replace(' ', '_')}={v.replace(' ', '_')}" for k, v in sorted(d.items()))
                    + "\n")
    # A kernel with a private (scratch) array or spilled vector registers
    # runs from memory that every access waits on: a silent slowdown of
    # several times. No kernel of the library may have either.
    bad = [(n, d.get("ScratchSize [bytes/lane]"), d.get("VGPRs Spill")) for n, d in res_all.items()
           if d.get("ScratchSize [bytes/lane]", "0") != "0" or d.get("VGPRs Spill", "0") != "0"]
    if bad:
        raise RuntimeError("kernels with scratch memory or spilled vector registers: " +
                           "; ".join(f"{n} (scratch {sc} B/lane, {sp} VGPRs spilled)" for n, sc, sp in bad))
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
