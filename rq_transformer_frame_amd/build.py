"""Build the HIP library (gfx950) in-tree with hipcc."""
from __future__ import annotations

import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libmoshi_mi355x.so")
CSRC = os.path.join(PKG, "csrc")
# translation units, compiled in parallel then linked (the persistent-kernel instances are the
# slow ones, split by head dim)
SOURCES = [os.path.join(CSRC, f) for f in (
    "moshi_api.hip", "persistent_hd128_bf16_kvf32.hip", "persistent_hd128_bf16_kvbf16.hip",
    "persistent_hd128_i8_kvf32.hip", "persistent_hd128_q4_kvf32.hip", "persistent_hd128_q8_kvf32.hip",
    "persistent_hd64.hip")]

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # no packed FP32 instructions in any kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-result",
]


def deps() -> list[str]:
    hdr = [os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".h")]
    return SOURCES + hdr + [os.path.join(ROOT, "include", "moshi_mi355x.h")]


def build(verbose: bool = False) -> str:
    """Compile every HIP source into libmoshi_mi355x.so (always recompiles)."""
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    tmp = LIB + ".tmp"
    objs, procs = [], []
    for src in SOURCES:
        obj = os.path.join(CSRC, os.path.basename(src)[:-4] + ".o")
        cmd = [hipcc, *HIPCC_FLAGS, "-I", os.path.join(ROOT, "include"), "-c", "-o", obj, src]
        if verbose:
            print(" ".join(cmd), flush=True)
        objs.append(obj)
        procs.append(subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True))
    errs = []
    for src, pr in zip(SOURCES, procs):
        _, err = pr.communicate()
        if pr.returncode != 0:
            errs.append(f"{os.path.basename(src)}:\n{err[-6000:]}")
    if errs:
        raise RuntimeError("hipcc failed:\n" + "\n".join(errs))
    cmd = [hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc link failed:\n" + res.stderr[-6000:])
    os.replace(tmp, LIB)
    for obj in objs:
        os.remove(obj)
    return LIB


def is_stale() -> bool:
    if not os.path.exists(LIB):
        return True
    t = os.path.getmtime(LIB)
    return any(os.path.getmtime(p) > t for p in deps())


if __name__ == "__main__":
    print(build(verbose=True))
