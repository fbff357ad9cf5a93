"""Build libkvc.so (HIP for gfx950) in-tree.

Every .hip file under csrc/ is compiled with hipcc to an object and the
objects are linked into compressed_decode_attention_gqa_amd/libkvc.so. Packed
fp32 VALU instructions are disabled for all device code.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
OUT = os.path.join(PKG, "libkvc.so")
BUILD_DIR = os.path.join(os.path.dirname(PKG), "_build")
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def common_flags(extra_defines=()):
    flags = ["-O3", "-std=c++17", f"--offload-arch={ARCH}", "-fPIC",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
             "-I", os.path.join(os.path.dirname(PKG), "include")]
    flags += [f"-D{d}" for d in extra_defines]
    return flags


def _compile(src: str, obj: str, defines) -> str:
    cmd = [hipcc(), "-c", src, "-o", obj] + common_flags(defines)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {os.path.basename(src)}:\n{r.stderr[-8000:]}")
    return r.stderr


def build(out: str = OUT, defines=(), verbose: bool = False, jobs: int = 8) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = sorted(f for f in os.listdir(CSRC) if f.endswith(".hip"))
    objs = [os.path.join(BUILD_DIR, os.path.splitext(f)[0] + ".o") for f in srcs]
    with cf.ThreadPoolExecutor(max_workers=min(jobs, len(srcs))) as ex:
        futs = [ex.submit(_compile, os.path.join(CSRC, s), o, defines) for s, o in zip(srcs, objs)]
        for f in futs:
            msg = f.result()
            if verbose and msg.strip():
                print(msg, file=sys.stderr)
    tmp = out + ".tmp"
    cmd = [hipcc(), "-shared", "-o", tmp, f"--offload-arch={ARCH}", "-fPIC"] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr[-8000:]}")
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
