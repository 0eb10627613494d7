"""Builds libkie.so in-tree with hipcc for gfx950 (no GPU needed)."""
from __future__ import annotations

import os
import shutil
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libkie.so")
SOURCES = ["kie_kernels.hip", "kie_prefill.hip", "kie_runtime.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def command(out: str = LIB, extra=()) -> list:
    return [hipcc(), "-O3", "-std=c++17", f"--offload-arch={ARCH}", "-fPIC", "-shared",
            # packed fp32 VALU ops stay off: plain fp32 code only
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wall", "-Wno-unused-function",
            "-I", os.path.join(ROOT, "include"), "-I", CSRC,
            *[os.path.join(CSRC, s) for s in SOURCES], *extra, "-o", out]


def build(verbose: bool = False, out: str = LIB, extra=()) -> str:
    cmd = command(out, extra)
    tmp = out + ".tmp"
    cmd[-1] = tmp
    res = subprocess.run(cmd, cwd=ROOT, capture_output=True, text=True)
    if verbose or res.returncode != 0:
        msg = "\n".join(l for l in (res.stdout + res.stderr).splitlines()
                        if "packed-fp32-ops" not in l and "is not a recognized feature" not in l)
        if msg.strip():
            print(msg)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed for libkie.so")
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
