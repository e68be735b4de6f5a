"""Compile the gfx950 HIP sources of this package into libattn.so, and the device-ceiling
probes (csrc/probes.hip, measurement only) into libattn_probes.so, both in the package folder.

Run ``python -m exact_softmax_attention_paged_amd.build`` or call ``build()``.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libattn.so")
SOURCES = ["attn_api.hip", "prefill_bf16.hip", "prefill_f32.hip", "decode_bf16.hip",
           "cascade_bf16.hip", "kv_write.hip", "schedule.hip"]
PROBES_LIB = os.path.join(PKG, "libattn_probes.so")
PROBES_SOURCES = ["probes.hip"]

# -packed-fp32-ops: no v_pk_{add,mul,fma}_f32 in the device code.
HIP_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Wno-unused-command-line-argument"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP library needs ROCm's hipcc to build")


def build(verbose: bool = False) -> str:
    """Always recompiles both libraries (each written atomically); returns libattn.so's path."""
    _compile(PROBES_SOURCES, PROBES_LIB, verbose)
    return _compile(SOURCES, LIB, verbose)


def _compile(sources, lib, verbose: bool) -> str:
    tmp = lib + ".tmp"
    cmd = [hipcc(), *HIP_FLAGS, "-I", INCLUDE, "-I", CSRC,
           *[os.path.join(CSRC, s) for s in sources], "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "'-packed-fp32-ops' is not a recognized feature"
    msg = "\n".join(l for l in (res.stdout + res.stderr).splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{msg}")
    if verbose and msg.strip():
        print(msg)
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
