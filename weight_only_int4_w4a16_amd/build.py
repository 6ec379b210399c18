"""Build libw4a16.so in-tree with hipcc for gfx950.

    python -m weight_only_int4_w4a16_amd.build [--jobs N] [extra hipcc flags]

Every HIP source is compiled with the packed-FP32 feature switched off
(-Xclang -target-feature -Xclang -packed-fp32-ops): ordinary float code only.
"""
from __future__ import annotations

import os
import shlex
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libw4a16.so")
SOURCES = ["kernels.hip", "kernels3.hip", "quantize.hip", "stream_probe.hip", "api.hip", "plan.cpp"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

COMMON = ["-O3", "-std=c++17", "-fPIC", "--offload-arch=gfx950",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-fhip-fp32-correctly-rounded-divide-sqrt",
          "-Wall", "-Wno-unused-function", "-I", INCLUDE, "-I", CSRC]


def build(out: str = LIB, extra=(), build_dir: str | None = None, jobs: int = 4) -> str:
    build_dir = build_dir or os.path.join(PKG, "_build")
    os.makedirs(build_dir, exist_ok=True)

    def compile_one(src):
        obj = os.path.join(build_dir, src + ".o")
        lang = ["-x", "hip"] if src.endswith(".hip") else ["-x", "c++"]
        cmd = [HIPCC, *COMMON, *extra, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed for {src}:\n{shlex.join(cmd)}\n{r.stderr}")
        return obj

    with ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = out + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{shlex.join(cmd)}\n{r.stderr}")
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    args = sys.argv[1:]
    jobs = 4
    if args[:1] == ["--jobs"]:
        jobs, args = int(args[1]), args[2:]
    print(build(extra=args, jobs=jobs))
