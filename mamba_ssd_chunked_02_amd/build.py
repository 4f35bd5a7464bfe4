"""Build step for libssd.so (the HIP kernels + C ABI), gfx950 only.

``python -m mamba_ssd_chunked_02_amd.build`` compiles the sources under
``csrc/`` with hipcc into ``libssd.so`` inside this package directory.
hipcc cross-compiles, so this runs on a machine without a GPU.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libssd.so")
SOURCES = ["ssd_api.hip", "ssd_kernels.hip", "ssd_hw_kernels.hip", "ssd_bwd_kernels.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# Packed-fp32 instructions are kept out of the device code (hipcc still
# forms ordinary VALU ops from float2 code); the host pass warns that it does
# not know the feature, which is harmless.
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-result",
]


def build(verbose: bool = False, extra=()) -> str:
    """Compile every source to an object in parallel (one hipcc each), then
    link the shared library."""
    from concurrent.futures import ThreadPoolExecutor

    obj_dir = os.path.join(ROOT, "_build")
    os.makedirs(obj_dir, exist_ok=True)
    inc = ["-I", os.path.join(ROOT, "include")]
    noise = "'-packed-fp32-ops' is not a recognized feature"
    compile_flags = [f for f in FLAGS if f != "-shared"]

    def run(cmd):
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
        return r.returncode, err

    objs, cmds = [], []
    for src in SOURCES:
        obj = os.path.join(obj_dir, src.replace(".hip", ".o"))
        objs.append(obj)
        cmds.append([HIPCC, *compile_flags, *extra, *inc, "-c", "-o", obj,
                     os.path.join(CSRC, src)])
    with ThreadPoolExecutor(max_workers=len(cmds)) as ex:
        results = list(ex.map(run, cmds))
    for (rc, err), cmd in zip(results, cmds):
        if rc != 0:
            raise RuntimeError(f"hipcc failed ({rc}) on {cmd[-1]}:\n{err}")
        if verbose and err.strip():
            print(err, file=sys.stderr)
    tmp = LIB + ".tmp"
    rc, err = run([HIPCC, *FLAGS, *extra, "-o", tmp, *objs])
    if rc != 0:
        raise RuntimeError(f"link failed ({rc}):\n{err}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
