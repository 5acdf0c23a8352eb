"""Build liblq.so (the HIP kernels and the C ABI) in-tree for gfx950.

    python -m bit_matmul_amd.build          # or bit_matmul_amd.build.build()

Every source under csrc/ is compiled with hipcc into _build/, then linked into
bit_matmul_amd/liblq.so. Always rebuilds (a few seconds per file, in parallel).
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor
from pathlib import Path

PKG = Path(__file__).resolve().parent
ROOT = PKG.parent
CSRC = PKG / "csrc"
BUILD = ROOT / "_build"
LIB = PKG / "liblq.so"
ARCH = os.environ.get("LQ_OFFLOAD_ARCH", "gfx950")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

COMMON = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17",
    # Keep the compiler from forming packed fp32 (v_pk_*_f32) instructions.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{ROOT / 'include'}", f"-I{CSRC}",
    "-Wall", "-Wno-unused-function",
]


def _sources():
    return sorted(list(CSRC.glob("*.hip")) + list(CSRC.glob("*.cpp")))


def _compile(src: Path) -> Path:
    obj = BUILD / (src.name + ".o")
    cmd = [HIPCC, *COMMON, "-c", str(src), "-o", str(obj)]
    if src.suffix == ".cpp":
        cmd = [HIPCC, *COMMON, "-x", "hip", "-c", str(src), "-o", str(obj)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msgs = [l for l in (res.stdout + res.stderr).splitlines() if noise not in l]
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src.name}:\n" + "\n".join(msgs))
    if msgs:
        sys.stderr.write("\n".join(msgs) + "\n")
    return obj


def build(verbose: bool = True) -> Path:
    BUILD.mkdir(exist_ok=True)
    srcs = _sources()
    with ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB.with_suffix(".so.tmp")
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *map(str, objs), "-o", str(tmp)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("link failed:\n" + res.stdout + res.stderr)
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB} from {len(srcs)} sources")
    return LIB


if __name__ == "__main__":
    build()
