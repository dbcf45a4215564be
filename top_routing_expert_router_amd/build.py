"""Build libmoe_mi355x.so (all HIP sources, gfx950) in-tree with hipcc.

Usage: python -m top_routing_expert_router_amd.build  (or build() from Python).
Each source compiles to an object in ``_build/``; the objects link into one
shared library next to this file.
"""
from __future__ import annotations

import concurrent.futures
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_NAME = "libmoe_mi355x.so"
LIB_PATH = os.path.join(HERE, LIB_NAME)
SOURCES = ["api.hip", "route.hip", "align.hip", "reroute.hip", "expert_choice.hip", "ffn.hip", "combine.hip"]
# measured hardware ceilings (copy / read streams, MFMA issue); not part of the layer
CEILING_LIB_PATH = os.path.join(HERE, "libmoe_ceiling.so")
CEILING_SOURCES = ["ceiling.hip"]
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
    # packed fp32 instructions are kept out of all device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


# per-source flags.  ffn.hip: the tile claims of the expert GEMMs are single-lane
# atomics whose result is needed only a whole tile later; the atomic optimizer would
# turn each into a wave-aggregated form that waits for the result at once.
SOURCE_FLAGS = {"ffn.hip": ["-mllvm", "-amdgpu-atomic-optimizer-strategy=None"]}


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, *SOURCE_FLAGS.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (res.stdout + res.stderr).splitlines()
                    if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{out}")
    if out.strip():
        sys.stderr.write(out + "\n")
    return obj


def _link(objs, path: str) -> None:
    tmp = path + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("link failed:\n" + res.stdout + res.stderr)
    os.replace(tmp, path)


def build(verbose: bool = False) -> str:
    """Compile every HIP source for gfx950 and link the shared libraries; returns the layer library's path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = SOURCES + CEILING_SOURCES
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(len(srcs), os.cpu_count() or 1)) as ex:
        objs = dict(zip(srcs, ex.map(_compile, srcs)))
    _link([objs[x] for x in SOURCES], LIB_PATH)
    _link([objs[x] for x in CEILING_SOURCES], CEILING_LIB_PATH)
    if verbose:
        print(f"built {LIB_PATH}")
        print(f"built {CEILING_LIB_PATH}")
    return LIB_PATH


if __name__ == "__main__":
    build(verbose=True)
