"""Build libhstu.so in-tree with hipcc for gfx950.

Every HIP translation unit is compiled with packed fp32 vector instructions
disabled (-Xclang -target-feature -Xclang -packed-fp32-ops); the host pass
warns that it does not know that feature, which is harmless.
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libhstu.so")
SOURCES = ["sched.hip", "attn_fwd.hip", "attn_bwd.hip", "norm.hip", "batching.hip", "layer.hip", "proj_gemm.hip", "gemm.cpp",
           "api.cpp", "static_ws.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-fPIC", "-std=c++17", "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I" + os.path.join(os.path.dirname(PKG), "include"),
]


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    procs = []
    objs = []
    for src in SOURCES:
        path = os.path.join(CSRC, src)
        if not os.path.exists(path):
            continue
        obj = os.path.join(BUILD, src + ".o")
        objs.append(obj)
        cmd = [HIPCC, *FLAGS, "-c", path, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
    failed = []
    for src, p in procs:
        out, _ = p.communicate()
        text = out.decode(errors="replace")
        text = "\n".join(l for l in text.splitlines()
                         if "packed-fp32-ops" not in l and "not a recognized feature" not in l)
        if p.returncode != 0:
            failed.append(src)
            sys.stderr.write(text + "\n")
        elif verbose and text.strip():
            sys.stderr.write(text + "\n")
    if failed:
        raise RuntimeError("hipcc failed for " + ", ".join(failed))
    tmp = LIB + ".tmp"
    subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs, "-L/opt/rocm/lib",
                    "-lhipblaslt", "-Wl,-rpath,/opt/rocm/lib"], check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
