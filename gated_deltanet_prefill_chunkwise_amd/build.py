"""Build libsgdn.so (the HIP kernels and the C ABI) for gfx950 with hipcc.

    python -m gated_deltanet_prefill_chunkwise_amd.build

Objects go to ``_build/`` at the repository root; the shared library is
written next to this file.  Every source is compiled with packed-fp32
instruction generation disabled; the selector is additionally compiled
without floating-point contraction (its decisions must be reproducible).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libsgdn.so")
BUILD = os.path.join(ROOT, "_build")

SOURCES = ["api.hip", "intra.hip", "hscan.hip", "ochunk.hip", "misc.hip", "select.hip",
           "decode.hip"]
# hscan: products accumulate in ordinary vector registers (its state tiles are
# also scaled and converted by vector instructions every event)
EXTRA = {"select.hip": ["-ffp-contract=off"],
         "hscan.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def common_flags(arch: str):
    return ["--offload-arch=" + arch, "-O3", "-std=c++17", "-fPIC",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", os.path.join(ROOT, "include"), "-I", CSRC]


def build(arch: str = "gfx950", verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    cc = hipcc()
    flags = common_flags(arch)

    def compile_one(src):
        obj = os.path.join(BUILD, src.replace(".hip", ".o"))
        cmd = [cc, *flags, *EXTRA.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed for {src}:\n{err}")
        if verbose and err.strip():
            print(err, file=sys.stderr)
        return obj

    with ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = OUT + ".tmp"
    cmd = [cc, "--offload-arch=" + arch, "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stderr)
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    print(build(verbose=True))
