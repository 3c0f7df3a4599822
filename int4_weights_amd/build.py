"""Build libmoe.so (the gfx950 HIP kernels and the C ABI) in-tree with hipcc.

    python -m int4_weights_amd.build        # or: from int4_weights_amd.build import build; build()
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OBJ = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libmoe.so")
SOURCES = ["api.hip", "quant.hip", "route.hip", "gemm_fp8.hip", "gemm_int4.hip", "gemm_bf16.hip", "gemm_fp4.hip",
           "gemm_int8.hip", "swiglu.hip", "combine.hip", "stream.hip"]
ARCH = os.environ.get("MOE_OFFLOAD_ARCH", "gfx950")


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (set HIPCC or install ROCm)")


def flags() -> list[str]:
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
        # packed fp32 VALU ops stay off (the kernels use plain fp32 math)
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wno-unused-command-line-argument",
        *os.environ.get("MOE_EXTRA_CFLAGS", "").split(),
    ]


def _compile(src: str) -> str:
    out = os.path.join(OBJ, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *flags(), "-c", os.path.join(CSRC, src), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return out


GENERATED = [("gen_fp8_asm.py", "gemm_fp8_tall_loop.inc")]


def generate() -> None:
    """Write the generated assembly includes (the tall FP8 main loop) next to the sources."""
    for script, out in GENERATED:
        r = subprocess.run([sys.executable, os.path.join(CSRC, script), os.path.join(CSRC, out)],
                           capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"{script} failed:\n{r.stderr}")


def build(verbose: bool = True) -> str:
    """Compile every HIP source for gfx950 and link libmoe.so; returns its path."""
    os.makedirs(OBJ, exist_ok=True)
    generate()
    jobs = min(len(SOURCES), int(os.environ.get("MAX_JOBS", os.cpu_count() or 4)))
    with ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), *flags(), "-shared", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}", file=sys.stderr)
    return LIB


if __name__ == "__main__":
    build()
