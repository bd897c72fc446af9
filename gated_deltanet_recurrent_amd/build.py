"""Build the gfx950 shared library ``libgdn_mi355x.so`` in-tree with hipcc.

    python -m gated_deltanet_recurrent_amd.build [--save-temps DIR]

Flags:
  --offload-arch=gfx950          MI355X (CDNA4) code object only
  -O3 -ffp-contract=off          no implicit FMA contraction: the kernels fuse
                                 exactly where they call an fma builtin, so the
                                 single-step, M-step and rollback instantiations
                                 compute identical bits
  -Xclang -target-feature -Xclang -packed-fp32-ops
                                 keep the compiler from emitting packed fp32
                                 (v_pk_*_f32) arithmetic
"""
from __future__ import annotations

import argparse
import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB_NAME = "libgdn_mi355x.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)
SOURCES = [os.path.join(CSRC, "gdn_kernels.hip"), os.path.join(CSRC, "gdn_api.cpp")]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-ffp-contract=off", "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


def build(verbose: bool = False, save_temps: str | None = None) -> str:
    tmp = LIB_PATH + ".tmp%d" % os.getpid()
    cmd = [HIPCC, *FLAGS, "-o", tmp, *SOURCES]
    if save_temps:
        os.makedirs(save_temps, exist_ok=True)
        cmd.insert(1, "-save-temps=obj")
        cmd = cmd[:]
        cwd = save_temps
    else:
        cwd = None
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True, cwd=cwd)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--save-temps", default=None, help="keep intermediate files (ISA) here")
    args = ap.parse_args()
    print(build(verbose=True, save_temps=args.save_temps))
