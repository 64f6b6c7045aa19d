"""Build libmoeffn.so (HIP, gfx950) in-tree with hipcc.

Run as ``python -m bit_gathered_quantized_amd.build``; ``__graft_entry__.build()``
calls :func:`build` as well.
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_PATH = os.path.join(PKG, "libmoeffn.so")
ARCH = "gfx950"

# -packed-fp32-ops: hipcc must not form packed fp32 instructions on its own.
HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Wall", "-Wextra", "-fno-fast-math",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA results straight into VGPRs: the per-group scale FMA reads them
    "-mllvm", "-amdgpu-mfma-vgpr-form",
]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def source_digest() -> str:
    """SHA-256 over the HIP sources, the public header and the build flags:
    identifies the kernels a measurement was taken on."""
    import hashlib
    h = hashlib.sha256(" ".join(HIPCC_FLAGS).encode())
    for path in sources() + sorted(glob.glob(os.path.join(CSRC, "*.h"))) + [
            os.path.join(INCLUDE, "moe_ffn.h")]:
        h.update(os.path.basename(path).encode())
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if err.strip() and verbose:
        print(err, file=sys.stderr)


def build(verbose: bool = False) -> str:
    """Compile every source to an object (in parallel), then link the shared
    library.  Objects go to a temporary folder; only the .so stays in-tree."""
    import tempfile
    from concurrent.futures import ThreadPoolExecutor
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    tmp = LIB_PATH + ".tmp"
    with tempfile.TemporaryDirectory(prefix="moeffn_build_") as d:
        objs, cmds = [], []
        for src in sources():
            obj = os.path.join(d, os.path.basename(src) + ".o")
            objs.append(obj)
            cmds.append([hipcc, *HIPCC_FLAGS, "-c", f"-I{INCLUDE}", f"-I{CSRC}", src, "-o", obj])
        jobs = max(1, min(len(cmds), os.cpu_count() or 1, 16))
        with ThreadPoolExecutor(jobs) as ex:
            list(ex.map(lambda c: _run(c, verbose), cmds))
        _run([hipcc, *HIPCC_FLAGS, "-shared", *objs, "-o", tmp], verbose)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
