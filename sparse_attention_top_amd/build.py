"""Build libsparse_mla.so (gfx950 only) in-tree with hipcc.

    python -m sparse_attention_top_amd.build            # build
    python -m sparse_attention_top_amd.build --resource # also print per-kernel VGPR/AGPR/LDS/occupancy
"""

from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRC = [os.path.join(PKG, "csrc", "sparse_mla.hip"), os.path.join(PKG, "csrc", "sparse_mla_bwd.hip")]
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libsparse_mla.so")
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=" + ARCH,
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Wall",
    # Packed fp32 VALU forms stay off: the compiler would otherwise emit them
    # from plain float code.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def build(resource_usage: bool = False) -> str:
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, *FLAGS, "-I", INCLUDE, "-o", tmp, *SRC]
    if resource_usage:
        cmd.insert(1, "-Rpass-analysis=kernel-resource-usage")
    proc = subprocess.run(cmd, capture_output=True, text=True)
    out = proc.stdout + proc.stderr
    # the host pass does not know the device feature above; that note is harmless
    out = "\n".join(line for line in out.splitlines() if "packed-fp32-ops" not in line)
    if proc.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + out)
    os.replace(tmp, LIB)
    if resource_usage and out.strip():
        print(out)
    return LIB


if __name__ == "__main__":
    build(resource_usage="--resource" in sys.argv)
    print(LIB)
