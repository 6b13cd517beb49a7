"""Build the HIP library ``libgemm18.so`` for gfx950 with hipcc, in-tree."""
from __future__ import annotations

import os
import shutil
import subprocess
from pathlib import Path

PKG = Path(__file__).resolve().parent
ROOT = PKG.parent
SRC = PKG / "csrc" / "gemm_nt_f16.hip"
HEADER = ROOT / "include" / "gemm_nt_f16.h"
LIB = PKG / "libgemm18.so"

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Wall",
    # Packed fp32 VALU forms stay off; hipcc's host pass warns that it does
    # not know the feature, which is harmless.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{ROOT / 'include'}",
]


def hipcc() -> str:
    found = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not Path(found).exists():
        raise RuntimeError("hipcc not found; the HIP library cannot be built")
    return found


def build(verbose: bool = False) -> Path:
    """Compile the library; always recompiles.  Returns the library path."""
    tmp = LIB.with_suffix(f".so.tmp{os.getpid()}")
    cmd = [hipcc(), *HIPCC_FLAGS, str(SRC), "-o", str(tmp)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{res.stderr}")
    if verbose and res.stderr:
        print(res.stderr)
    os.replace(tmp, LIB)
    return LIB


def stale() -> bool:
    """True if the library is missing or older than its sources."""
    if not LIB.exists():
        return True
    t = LIB.stat().st_mtime
    return any(p.stat().st_mtime > t for p in (SRC, HEADER))


if __name__ == "__main__":
    print(build(verbose=True))
