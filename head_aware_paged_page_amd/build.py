"""Build libsegpaged.so (HIP for gfx950) in-tree with hipcc."""
from __future__ import annotations

import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB_DIR = os.path.join(PKG, "_lib")
LIB = os.path.join(LIB_DIR, "libsegpaged.so")
SOURCES = ["tables.cpp", "runtime.cpp", "relocate.hip", "prefill.hip", "decode.hip", "attn_f32.hip", "pack.hip", "noalloc.hip", "importance.hip"]
ARCH = "gfx950"


def hipcc_cmd(out: str = LIB):
    return ["hipcc", "-x", "hip", f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wno-unused-command-line-argument", f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}",
            *[os.path.join(CSRC, s) for s in SOURCES], "-o", out]


def build(verbose: bool = False) -> str:
    """Compile every source into libsegpaged.so (always recompiles)."""
    os.makedirs(LIB_DIR, exist_ok=True)
    tmp = LIB + ".tmp"
    cmd = hipcc_cmd(tmp)
    res = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in res.stderr.splitlines() if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{' '.join(cmd)}\n{err}")
    if verbose and err.strip():
        print(err)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
