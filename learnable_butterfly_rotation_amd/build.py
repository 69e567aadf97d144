"""Build libbfly.so (HIP, gfx950) in-tree with hipcc.

Usage: python -m learnable_butterfly_rotation_amd.build
Each translation unit is compiled in parallel, then linked into a shared
library next to this file.
"""
from __future__ import annotations

import os
import subprocess
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OBJ = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libbfly.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# (source, object, extra flags): the Kronecker unit is compiled once per m
SOURCES = [("bfly_api.hip", "bfly_api.o", []), ("bfly_bwd.hip", "bfly_bwd.o", []),
           ("bfly_fwd_plain.hip", "bfly_fwd_plain.o", []),
           ("bfly_qgemm.hip", "bfly_qgemm.o", []),
           ("bfly_kron_bwd.hip", "bfly_kron_bwd.o", []),
           ("bfly_kron_mix.hip", "bfly_kron_mix.o", []),
           ("bfly_calib.hip", "bfly_calib.o", []),
           ("bfly_calib_w.hip", "bfly_calib_w.o", []),
           ("bfly_fwd8k.hip", "bfly_fwd8k.o", []),
           ("bfly_kron_fused.hip", "bfly_kron_fused.o", [])] + \
          [("bfly_fwd_kron.hip", "bfly_fwd_kron_m%d.o" % m, ["-DKRON_M=%d" % m]) for m in range(2, 9)]

FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "--offload-arch=gfx950",
    # no packed fp32 (v_pk_*_f32) code generation
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # NaN inputs give unspecified results; min/max then need no NaN quieting
    "-fno-honor-nans",
    "-Wall", "-Wno-unused-function",
]


def build(verbose: bool = False, extra=None) -> str:
    os.makedirs(OBJ, exist_ok=True)
    t0 = time.time()
    procs = []
    for src, objname, defs in SOURCES:
        obj = os.path.join(OBJ, objname)
        cmd = [HIPCC, *FLAGS, *defs, *(extra or []), "-c", os.path.join(CSRC, src), "-o", obj]
        procs.append((src, obj, subprocess.Popen(cmd, stdout=subprocess.PIPE,
                                                 stderr=subprocess.STDOUT, text=True)))
    objs, failed = [], []
    for src, obj, p in procs:
        out, _ = p.communicate()
        if verbose and out.strip():
            print(out, file=sys.stderr)
        if p.returncode != 0:
            failed.append((src, out))
        objs.append(obj)
    if failed:
        for src, out in failed:
            print("---- %s ----\n%s" % (src, out), file=sys.stderr)
        raise RuntimeError("hipcc failed for: " + ", ".join(s for s, _ in failed))
    tmp = LIB + ".tmp%d" % os.getpid()
    subprocess.run([HIPCC, "-shared", "-fPIC", "--offload-arch=gfx950", *objs, "-o", tmp],
                   check=True)
    os.replace(tmp, LIB)
    if verbose:
        print("built %s in %.1f s" % (LIB, time.time() - t0), file=sys.stderr)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
