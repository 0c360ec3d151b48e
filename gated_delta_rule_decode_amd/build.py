"""Build libgdn.so in-tree with hipcc for gfx950.

    python -m gated_delta_rule_decode_amd.build

Compiles every source under csrc/ to an object (in parallel) and links the
shared library next to this file.  Device code is built for gfx950 only, with
packed-fp32 instruction selection turned off and MFMA results kept in VGPRs.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIBRARY = os.path.join(PKG, "libgdn.so")
SOURCES = ["gdn_api.cpp", "gdn_attn.hip", "gdn_decode.hip", "gdn_noalloc.hip", "gdn_prefill.hip",
           "gdn_prefill_mfma.hip", "gdn_prefill_tp.hip", "gdn_rmsnorm.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def common_flags():
    return ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", INCLUDE, "-I", CSRC,
            "-Wall", "-Wno-unused-function", "-Wno-unused-command-line-argument",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-ffp-contract=fast",
            # MFMA accumulators in ordinary VGPRs: results feed vector code
            # directly, without accumulator-register copies
            "-mllvm", "-amdgpu-mfma-vgpr-form=1"]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *common_flags(), "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {src}\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    warn = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l
                     and "not a recognized feature" not in l).strip()
    if warn:
        sys.stderr.write(warn + "\n")
    return obj


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIBRARY + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIBRARY)
    if verbose:
        print(f"built {LIBRARY}")
    return LIBRARY


if __name__ == "__main__":
    build()
