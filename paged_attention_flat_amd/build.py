"""Build libpa.so (the HIP kernels and the C ABI) in-tree for gfx950.

Run as ``python paged_attention_flat_amd/build.py`` or through
``__graft_entry__.build()``.  Compiles every time it is called.  This file
imports nothing from the package (whose import loads the built library).
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libpa.so")
SOURCES = ["kv_write.hip", "decode.hip", "prefill.hip", "attn_f32.hip", "combine.hip",
           "mixed.hip", "pa_api.cpp", "noalloc.cpp"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
# Packed fp32 instructions are kept off for every kernel (hipcc -O3 would
# otherwise form them from scalar float code).
FLAGS = ["-O3", "-std=c++17", "-fPIC", "--offload-arch=gfx950",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wno-unused-command-line-argument", "-I" + os.path.join(ROOT, "include")]

# Per-file additions.  The prefill kernel reduces row maxima of MFMA results,
# which IEEE mode would first quiet (one extra v_max per value); its inputs to
# max are finite or -inf by construction (masked scores are selected to -inf,
# keys past the context are zero-filled before use), so it is built without
# NaN semantics and with the IEEE mode bit off.
SOURCE_FLAGS = {"prefill.hip": ["-fno-honor-nans", "-mno-amdgpu-ieee"]}


def build(verbose: bool = False) -> str:
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    objs = []
    procs = []
    for src in SOURCES:
        obj = os.path.join(objdir, os.path.splitext(src)[0] + ".o")
        lang = ["-x", "hip"] if src.endswith(".cpp") else []
        cmd = [HIPCC, *FLAGS, *SOURCE_FLAGS.get(src, []), *lang, "-c", os.path.join(CSRC, src),
               "-o", obj]
        procs.append((src, cmd, subprocess.Popen(cmd, stdout=subprocess.PIPE,
                                                  stderr=subprocess.STDOUT, text=True)))
        objs.append(obj)
    failed = []
    for src, cmd, p in procs:
        out, _ = p.communicate()
        if verbose or p.returncode != 0:
            sys.stderr.write(out)
        if p.returncode != 0:
            failed.append(src)
    if failed:
        raise RuntimeError("hipcc failed for " + ", ".join(failed))
    tmp = LIB + ".tmp"
    link = [HIPCC, "-shared", "-fPIC", "--offload-arch=gfx950", "-o", tmp, *objs]
    subprocess.run(link, check=True)
    os.replace(tmp, LIB)
    shutil.rmtree(objdir, ignore_errors=True)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
