"""Build libwq.so for gfx950 with hipcc, in the source tree.

    python -m dequant_gemv_rht_amd.build          # compile every source, link
    python -m dequant_gemv_rht_amd.build --asm    # also keep the AMD assembly

Each source file compiles to its own object in parallel; the library lands
in ``dequant_gemv_rht_amd/_lib/libwq.so``.
"""

from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "_lib")
LIB = os.path.join(OUT, "libwq.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

COMMON = [
    "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
    f"--offload-arch={ARCH}",
    # keep the compiler from forming packed fp32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp")))


def _compile(src: str, asm: bool) -> str:
    obj = os.path.join(OUT, os.path.basename(src) + ".o")
    cmd = [HIPCC] + COMMON + ["-c", src, "-o", obj]
    if src.endswith(".hip"):
        cmd[1:1] = ["-x", "hip"]
        if os.path.basename(src) == "gemv_stream.hip":
            # the GEMV kernels' first seven arguments (the linears' first
            # workgroups) arrive preloaded in scalar registers
            cmd += ["-mllvm", "-amdgpu-kernarg-preload-count=7"]
        if asm:
            cmd += ["-save-temps=obj"]
    r = subprocess.run(cmd, capture_output=True, text=True, cwd=OUT)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


def build(asm: bool = False, jobs: int | None = None) -> str:
    os.makedirs(OUT, exist_ok=True)
    srcs = sources()
    jobs = jobs or min(len(srcs), max(1, (os.cpu_count() or 4)))
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, asm), srcs))
    tmp = LIB + ".tmp%d" % os.getpid()
    r = subprocess.run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs,
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(asm="--asm" in sys.argv))
