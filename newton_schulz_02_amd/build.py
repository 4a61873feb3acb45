"""Build ``libmuon.so`` (HIP kernels for gfx950 + the C ABI) in-tree with hipcc.

Usage:  python -m newton_schulz_02_amd.build  [--verbose]

Each source is compiled to an object under ``newton_schulz_02_amd/_build`` in parallel,
then linked into ``newton_schulz_02_amd/libmuon.so``.  Packed-fp32 instruction
generation is disabled for all device code.
"""

from __future__ import annotations

import hashlib
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor
from pathlib import Path

PKG = Path(__file__).resolve().parent
ROOT = PKG.parent
CSRC = PKG / "csrc"
BUILD = PKG / "_build"
LIB = PKG / "libmuon.so"
ARCH = "gfx950"

SOURCES = ["planner.cpp", "shampoo_plan.cpp", "muon_api.cpp", "owner.cpp", "kernels_elementwise.hip", "kernels_gemm.hip",
           "kernels_gemm_wide.hip", "noalloc.hip"]
# Sources compiled a second time with extra defines: (source, object stem, flags).
VARIANTS = [("kernels_gemm.hip", "kernels_gemm_deep", ["-DMUON_GEMM_DEEP=1"]),
            ("kernels_gemm.hip", "kernels_gemm_small", ["-DMUON_GEMM_SMALL=1"])]
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def kernel_hash() -> str:
    """Hash of the device sources (every .hip and .h file under csrc), 16 hex digits.

    Compiled into the library (muon_kernel_hash); a tuning table records the hash of the
    kernels it was measured on, and a library built from other sources refuses it."""
    h = hashlib.sha256()
    for p in sorted(CSRC.glob("*.hip")) + sorted(CSRC.glob("*.h")):
        h.update(p.name.encode())
        h.update(p.read_bytes())
    return h.hexdigest()[:16]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and Path(cand).exists():
            return cand
    raise RuntimeError("hipcc not found (set HIPCC or install ROCm)")


def _compile(src: Path, obj: Path, verbose: bool, khash: str, extra=()) -> None:
    cmd = [hipcc(), "-O3", "-std=c++17", "-fPIC", "-Wall", f"-I{ROOT / 'include'}", f"-I{CSRC}",
           f'-DMUON_KERNEL_HASH="{khash}"', *extra]
    if src.suffix == ".hip":
        cmd += ["-x", "hip", f"--offload-arch={ARCH}", *DEVICE_FLAGS]
    else:
        cmd += ["-D__HIP_PLATFORM_AMD__"]
    cmd += ["-c", str(src), "-o", str(obj)]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    out = (res.stdout + res.stderr).strip()
    # hipcc's host pass warns that it does not know the packed-fp32 feature; drop that noise.
    lines = [ln for ln in out.splitlines() if "packed-fp32-ops" not in ln and ln.strip()]
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src.name}:\n" + "\n".join(lines))
    if verbose and lines:
        print("\n".join(lines), flush=True)


def build(verbose: bool = False) -> Path:
    BUILD.mkdir(exist_ok=True)
    jobs = [(CSRC / s, BUILD / (Path(s).stem + ".o"), ()) for s in SOURCES]
    jobs += [(CSRC / s, BUILD / (stem + ".o"), tuple(flags)) for s, stem, flags in VARIANTS]
    objs = [o for _, o, _ in jobs]
    khash = kernel_hash()
    with ThreadPoolExecutor(max_workers=len(jobs)) as ex:
        futs = [ex.submit(_compile, src, o, verbose, khash, extra) for src, o, extra in jobs]
        for f in futs:
            f.result()
    tmp = LIB.with_suffix(".so.tmp")
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", str(tmp), *map(str, objs)]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("link failed:\n" + res.stdout + res.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    path = build(verbose="--verbose" in sys.argv)
    print(path)
