"""Build the gfx950 shared library libdcpattn.so in-tree (hipcc, no JIT)."""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libdcpattn.so")
SOURCES = ["dcp_api.cpp", "noalloc.hip", "plan.hip", "merge.hip", "gqa_shard.hip",
           "gqa_fp8.hip", "mla_shard.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall",
         # packed fp32 VALU forms are kept out of the generated code
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", INCLUDE, "-I", CSRC]


# Per-source flags.  mla_shard.hip: MFMA builtins keep their accumulators in VGPRs (its
# AGPRs are all taken by inline-asm accumulators).
EXTRA_FLAGS = {"mla_shard.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}

# The host pass of hipcc does not know the target feature named in FLAGS and says so once
# per source; that line is the only compiler output a clean build may print.
_BENIGN = ("packed-fp32-ops",)


def _compile(src):
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC] + FLAGS + EXTRA_FLAGS.get(src, []) + ["-x", "hip", "-c", os.path.join(CSRC, src),
                                                        "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                    if not any(b in l for b in _BENIGN))
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{out}")
    return obj, out


def build(allow_warnings=False):
    """Compile every source for gfx950 and link libdcpattn.so next to this file.

    Compiler warnings are printed and fail the build (-Wall is on), unless allow_warnings
    (or DCP_ALLOW_WARNINGS=1) is set, in which case they are only printed."""
    os.makedirs(BUILD, exist_ok=True)
    jobs = min(len(SOURCES), int(os.environ.get("MAX_JOBS", "8")))
    with ThreadPoolExecutor(jobs) as ex:
        results = list(ex.map(_compile, SOURCES))
    warned = [(src, out) for src, (_, out) in zip(SOURCES, results) if out.strip()]
    for src, out in warned:
        print(f"--- compiler output for {src}:\n{out}", file=sys.stderr)
    allow_warnings = allow_warnings or os.environ.get("DCP_ALLOW_WARNINGS") == "1"
    if warned and not allow_warnings:
        raise RuntimeError("compiler warnings in " + ", ".join(s for s, _ in warned) +
                           " (set DCP_ALLOW_WARNINGS=1 to build anyway)")
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + [o for o, _ in results]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(allow_warnings="--allow-warnings" in sys.argv))
