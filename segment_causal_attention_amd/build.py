"""Build libnomas.so (HIP, gfx950 only) in-tree with hipcc.

Each translation unit is compiled to an object under _build/ (in parallel),
then linked into segment_causal_attention_amd/libnomas.so.  Packed-fp32 VALU
instructions are disabled for all device code.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libnomas.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SOURCES = ["api.hip", "rope_tables.hip", "kv_quant.hip", "rope3d.hip", "seg_attn.hip", "cam_xattn.hip", "w8a16.hip",
           "seg_attn_bwd.hip"]
# The attention kernels take maxima with v_max/v_max3; without IEEE mode they
# need no NaN-quieting copies of every operand.  NaN inputs still propagate to
# every row that can see them through the products.
PER_FILE = {"seg_attn.hip": ["-fno-honor-nans", "-mno-amdgpu-ieee"],
            "cam_xattn.hip": ["-fno-honor-nans", "-mno-amdgpu-ieee"]}
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wno-unused-command-line-argument"]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # hipcc's host pass does not know the packed-fp32 feature and says so; drop that line
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError("command failed: %s\n%s" % (" ".join(cmd), out))
    return out


def build(verbose: bool = False, extra_flags=()) -> str:
    os.makedirs(BUILD, exist_ok=True)
    objs = []
    cmds = []
    for s in SOURCES:
        o = os.path.join(BUILD, s.replace(".hip", ".o"))
        objs.append(o)
        cmds.append([HIPCC, *FLAGS, *PER_FILE.get(s, []), *extra_flags, "-I", INCLUDE, "-c",
                     os.path.join(CSRC, s), "-o", o])
    with ThreadPoolExecutor(min(len(cmds), os.cpu_count() or 1)) as ex:
        outs = list(ex.map(_run, cmds))
    tmp = LIB + ".tmp%d" % os.getpid()
    link = _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp])
    os.replace(tmp, LIB)
    if verbose:
        for o in outs + [link]:
            if o.strip():
                print(o)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
