"""Build liblsreplay.so in-tree with hipcc for gfx950 (usable without a GPU: hipcc cross-compiles)."""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "liblsreplay.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

HIP_SOURCES = ["grpo_loss.hip", "replay_attn_fwd.hip", "replay_attn_bwd.hip", "replay_attn_dq.hip", "replay_attn_dkdv.hip", "pack.hip",
               "replay_attn_wide_fwd.hip", "replay_attn_wide_bwd.hip", "noalloc.hip", "lmhead.hip",
               "replay_attn_dkdv64.hip"]
CXX_SOURCES = ["api.cpp", "attn_plan.cpp", "timer.cpp"]
COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function", "-I", os.path.join(ROOT, "include")]
# the packed-fp32 feature stays off: every v_pk_*_f32 is left out of the kernels
HIP_FLAGS = ["--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-ffp-contract=fast"]
# Per-source extras. Forward and dQ: MFMA results in VGPRs -- their score tiles are read by VALU
# ops, which cannot address AGPRs, and the default AGPR form copies them back and forth.
SOURCE_FLAGS = {"replay_attn_fwd.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
                "replay_attn_dq.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
                "replay_attn_dkdv.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
                "replay_attn_dkdv64.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
                "replay_attn_wide_fwd.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def _run(cmd):
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # the host pass does not know the packed-fp32 target feature; that warning is harmless
    out = "\n".join(line for line in p.stdout.splitlines() if "packed-fp32-ops" not in line)
    if p.returncode != 0:
        raise RuntimeError(f"command failed ({p.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build(verbose: bool = False, extra_flags: list[str] | None = None) -> str:
    os.makedirs(BUILD, exist_ok=True)
    extra = list(extra_flags or [])
    jobs = []
    for s in HIP_SOURCES:
        obj = os.path.join(BUILD, s + ".o")
        jobs.append([HIPCC, *COMMON, *HIP_FLAGS, *SOURCE_FLAGS.get(s, []), *extra, "-c", os.path.join(CSRC, s),
                     "-o", obj])
    for s in CXX_SOURCES:
        obj = os.path.join(BUILD, s + ".o")
        jobs.append([HIPCC, *COMMON, *extra, "-D__HIP_PLATFORM_AMD__", "-I", "/opt/rocm/include", "-x", "c++", "-c", os.path.join(CSRC, s), "-o", obj])
    with ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        outs = list(ex.map(_run, jobs))
    if verbose:
        for o in outs:
            if o.strip():
                print(o)
    # ISA check of every device object (see isa_check.py)
    sys.path.insert(0, PKG)
    import isa_check
    asm_jobs = []
    for s in HIP_SOURCES:
        asm = os.path.join(BUILD, s + ".s")
        asm_jobs.append([HIPCC, *COMMON, *HIP_FLAGS, *SOURCE_FLAGS.get(s, []), *extra, "-S", "--cuda-device-only",
                         os.path.join(CSRC, s), "-o", asm])
    with ThreadPoolExecutor(max_workers=min(8, len(asm_jobs))) as ex:
        list(ex.map(_run, asm_jobs))
    for j in asm_jobs:
        text = open(j[-1]).read()
        bad = isa_check.scan(text) + isa_check.loop_scratch(text)
        if bad:
            raise RuntimeError(f"ISA check failed for {j[-1]}:\n" + "\n".join(bad[:20]))
    objs = [j[-1] for j in jobs]
    tmp = LIB + ".tmp"
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
