"""Build libspecverify.so (HIP, gfx950) in-tree with hipcc."""

from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libspecverify.so")
SOURCES = ["api.hip", "attention.hip", "reject.hip", "commit.hip", "upstream.hip"]
ARCH = "gfx950"

# -packed-fp32-ops: keep the compiler from forming packed fp32 VALU instructions.
HIPFLAGS = ["-O3", "-std=c++17", f"--offload-arch={ARCH}", "-fPIC",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wall", "-Wno-unused-function",
            f"-I{INCLUDE}", f"-I{CSRC}"]


# Per-file flags. Attention: keep the MFMA accumulators in VGPRs (the MFMA's VGPR form).
# Left to its heuristic, the compiler chose the AGPR form for the P.V products and then,
# because the online softmax rescales those accumulators with VALU multiplies, copied
# every accumulator from AGPRs to VGPRs and back on each 32-key block: 72 copies per
# block in the one-tile kernel, 144 in the two-tile one. With the VGPR form the key loop
# has none, the one-tile kernel needs no AGPRs at all, and the outputs are the same bits
# (7B shape at B = 256: 327.5 us instead of 334.8 us; 8B 203.6 instead of 205.5). The LM
# head, whose accumulators are never touched by VALU in its loop, keeps the default.
FILE_FLAGS = {"attention.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}


def hipcc() -> str:
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(exe):
        raise RuntimeError("hipcc not found; install ROCm or put hipcc on PATH")
    return exe


def _compile(src: str, obj: str) -> None:
    cmd = [hipcc(), *HIPFLAGS, *FILE_FLAGS.get(os.path.basename(src), []), "-c", src, "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(line for line in res.stderr.splitlines() if noise not in line)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{err}")
    if err.strip():
        sys.stderr.write(err + "\n")


def build(verbose: bool = True) -> str:
    objdir = os.path.join(PKG, "_build")
    os.makedirs(objdir, exist_ok=True)
    jobs = []
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        for s in SOURCES:
            src = os.path.join(CSRC, s)
            obj = os.path.join(objdir, s.replace(".hip", ".o"))
            jobs.append(ex.submit(_compile, src, obj))
        for j in jobs:
            j.result()
    objs = [os.path.join(objdir, s.replace(".hip", ".o")) for s in SOURCES]
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("link failed:\n" + res.stderr)
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build()
