"""Build the HIP library ``libgemm18.so`` for gfx950 with hipcc, in-tree."""
from __future__ import annotations

import os
import shutil
import subprocess
from pathlib import Path

PKG = Path(__file__).resolve().parent
ROOT = PKG.parent
CSRC = PKG / "csrc"
# One translation unit per entry-point family; they share gemm_kernels.h and
# compile in parallel.
SOURCES = [CSRC / "gemm_nt_f16.hip", CSRC / "gemm_nt_f16_ex.hip", CSRC / "gemm_nt_bf16.hip",
           CSRC / "gemm_nt_fp8.hip", CSRC / "gemm_nt_fp8_b5.hip", CSRC / "gemm_nt_f16_noalloc.hip",
           CSRC / "gemm_nt_f16_acc16.hip"]
HEADERS = [CSRC / "gemm_kernels.h", CSRC / "gemm_fp8.h", ROOT / "include" / "gemm_nt_f16.h"]
LIB = PKG / "libgemm18.so"

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
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
    """Compile every translation unit (in parallel) and link the library;
    always recompiles.  Returns the library path."""
    tag = f"tmp{os.getpid()}"
    objs = [LIB.with_name(f"{src.stem}.{tag}.o") for src in SOURCES]
    procs = [subprocess.Popen([hipcc(), *HIPCC_FLAGS, "-c", str(src), "-o", str(obj)],
                              stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)
             for src, obj in zip(SOURCES, objs)]
    errors = []
    for src, proc in zip(SOURCES, procs):
        _, err = proc.communicate()
        if proc.returncode != 0:
            errors.append(f"{src.name}: hipcc failed ({proc.returncode}):\n{err}")
        elif verbose and err:
            print(err)
    try:
        if errors:
            raise RuntimeError("\n".join(errors))
        tmp = LIB.with_suffix(f".so.{tag}")
        res = subprocess.run([hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC",
                              *map(str, objs), "-o", str(tmp)], capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError(f"link failed ({res.returncode}):\n{res.stderr}")
        os.replace(tmp, LIB)
    finally:
        for obj in objs:
            if obj.exists():
                obj.unlink()
    return LIB


def stale() -> bool:
    """True if the library is missing or older than its sources."""
    if not LIB.exists():
        return True
    t = LIB.stat().st_mtime
    return any(p.stat().st_mtime > t for p in (*SOURCES, *HEADERS))


if __name__ == "__main__":
    print(build(verbose=True))
