"""Compile the HIP sources of the library into int4_expert_routing_amd/libmoe_q4.so (gfx950)."""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
LIB_NAME = "libmoe_q4.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)
SOURCES = ["route.hip", "gemm_q4.hip", "rows.hip", "decode_q4.hip", "quant_q4.hip", "moe_abi.hip"]
ARCH = "gfx950"


def hipcc_path() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def compile_command(out: str = LIB_PATH, extra=()) -> list:
    return [hipcc_path(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
            # keep the compiler from emitting packed fp32 arithmetic
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wno-unused-command-line-argument",
            "-I", os.path.join(ROOT, "include"),
            *[os.path.join(CSRC, s) for s in SOURCES], *extra, "-o", out]


def build(verbose: bool = False) -> str:
    tmp = LIB_PATH + ".tmp"
    cmd = compile_command(tmp)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed with status {res.returncode}")
    if verbose:
        # the host pass warns that it does not know the packed-fp32 feature; drop that line
        msg = "\n".join(l for l in (res.stdout + res.stderr).splitlines() if "packed-fp32-ops" not in l)
        if msg.strip():
            sys.stderr.write(msg + "\n")
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
