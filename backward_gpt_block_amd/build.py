"""Compile the HIP library (csrc/blk.hip, csrc/attn.hip) for gfx950 into this
package: ``libblk.so`` next to this file.  hipcc cross-compiles without a GPU."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libblk.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 VALU forms stay off: plain scalar fp32 instructions only
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-result", "-Wno-unused-value",
]

# translation units and their extra flags.  The attention kernels keep MFMA
# results in vector registers: their score blocks feed vector arithmetic, and
# the default placement in accumulation registers copied them back and forth.
UNITS = [
    ("blk.hip", []),
    ("attn.hip", ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]),
]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    errs = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{errs}")


def build(verbose: bool = False) -> str:
    """Compile every HIP translation unit and link libblk.so (always
    recompiles)."""
    objs = []
    for src, extra in UNITS:
        obj = os.path.join(HERE, src.replace(".hip", ".o"))
        _run([HIPCC, *FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj], verbose)
        objs.append(obj)
    tmp = OUT + ".tmp"
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
    os.replace(tmp, OUT)
    for obj in objs:
        os.remove(obj)
    return OUT


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
