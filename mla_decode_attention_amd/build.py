"""Build libmla_decode.so in-tree with hipcc for gfx950.

    python -m mla_decode_attention_amd.build
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB_NAME = "libmla_decode.so"
DEBUG_LIB_NAME = "libmla_decode_debug.so"   # MLA_DEBUG_BOUNDS: page ids checked against the pool
SOURCES = ["csrc/mla_kernels.hip", "csrc/mla_append.hip", "csrc/mla_prefill.hip", "csrc/mla_api.hip",
           "csrc/mla_scratch.hip", "csrc/mla_decode_so.hip", "csrc/mla_prefill_q8.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    return "hipcc"


def build(verbose: bool = True, debug_bounds: bool = False) -> str:
    out = os.path.join(HERE, DEBUG_LIB_NAME if debug_bounds else LIB_NAME)
    tmp = out + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
           # no packed-fp32 VALU forms (v_pk_fma_f32 & co.) in device code
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           # MFMA accumulators in VGPRs: the softmax rescale and the epilogue
           # then touch O without AGPR<->VGPR copies
           "-mllvm", "-amdgpu-mfma-vgpr-form=1",
           "-Wno-unused-result",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(HERE, "csrc")]
    if debug_bounds:
        cmd += ["-DMLA_DEBUG_BOUNDS"]
    cmd += [os.path.join(HERE, s) for s in SOURCES]
    cmd += ["-o", tmp]
    if verbose:
        print("[build]", " ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msg = "\n".join(l for l in (res.stdout + res.stderr).splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{msg}")
    if verbose and msg.strip():
        print(msg, flush=True)
    os.replace(tmp, out)
    return out


def build_all(verbose: bool = True):
    """The release library and the MLA_DEBUG_BOUNDS one."""
    return build(verbose), build(verbose, debug_bounds=True)


if __name__ == "__main__":
    for path in (build_all() if "--debug" in sys.argv else (build(),)):
        print(path)
    sys.exit(0)
