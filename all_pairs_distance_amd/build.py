"""Compile the HIP sources into the in-tree shared library libdbscan.so.

    python -m all_pairs_distance_amd.build

gfx950 only.  Flags that matter for the results:
  -ffp-contract=off                 every +, - and * of the distance is
                                    rounded on its own (no multiply-add);
  -fno-gpu-flush-denormals-to-zero  subnormal squares are kept;
  -Xclang -target-feature -Xclang -packed-fp32-ops
                                    no packed fp32 instructions are formed.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libdbscan.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = ["api.hip", "k_count.hip", "k_count_mfma.hip", "k_prep.hip",
           "k_merge.hip", "k_prune.hip", "k_relabel.hip", "k_graph.hip",
           "k_screen.hip"]
HEADERS = ["internal.h", "device.h", "count_common.h"]
ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-ffp-contract=off", "-fno-gpu-flush-denormals-to-zero",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
    f"-I{os.path.join(ROOT, 'include')}",
]


def _run(cmd):
    p = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the gfx feature name: harmless warning
    err = "\n".join(line for line in p.stderr.splitlines()
                    if "packed-fp32-ops" not in line
                    and "unknown target feature" not in line)
    if p.returncode != 0:
        raise RuntimeError(f"command failed: {' '.join(cmd)}\n{err}")
    return err


def build(verbose: bool = False) -> str:
    """Always recompiles; returns the library path."""
    os.makedirs(BUILD, exist_ok=True)
    objs = []
    jobs = []
    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), 8)) as ex:
        for src in SOURCES:
            obj = os.path.join(BUILD, src.replace(".hip", ".o"))
            objs.append(obj)
            cmd = [HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
            jobs.append(ex.submit(_run, cmd))
        for j in jobs:
            msg = j.result()
            if verbose and msg.strip():
                print(msg, file=sys.stderr)
    tmp = LIB + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs])
    os.replace(tmp, LIB)
    return LIB


def device_assembly(out: str, src: str = "k_count.hip") -> str:
    """Write the gfx950 assembly of one source (for instruction checks)."""
    _run([HIPCC, *FLAGS, "--cuda-device-only", "-S",
          os.path.join(CSRC, src), "-o", out])
    return out


if __name__ == "__main__":
    print(build(verbose=True))
