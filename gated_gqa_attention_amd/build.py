"""Build libqsa.so (the HIP kernels and the C ABI) in-tree for gfx950.

    python -m gated_gqa_attention_amd.build

Every translation unit is compiled separately (in parallel) into _build/ and
linked into gated_gqa_attention_amd/libqsa.so.  Packed fp32 VALU instructions
are disabled for all device code.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libqsa.so")
BUILD = os.path.join(ROOT, "_build")
SOURCES = ["qsa_api.hip", "qsa_rows.hip", "qsa_stream.hip", "qsa_prefill.hip", "qsa_merge.hip", "qsa_linear.hip",
           "qsa_turbo.hip", "qsa_gdn.hip"]
# per-source extra flags: the streaming, tile and merge kernels take their leading
# argument dwords (metadata and query pointers, grid shape) preloaded into
# SGPRs; their LDS copies set M0 from inline assembly, hence -Wno-inline-asm
# (nothing else in those files uses M0).  The short-query kernel keeps its MFMA
# accumulators in VGPRs (-amdgpu-mfma-vgpr-form): it fits in the 512 registers
# of one wavefront per SIMD, and AGPR accumulators cost a copy of every output
# register per key stage.
EXTRA = {"qsa_stream.hip": ["-mllvm", "-amdgpu-kernarg-preload-count=13", "-mllvm", "-amdgpu-mfma-vgpr-form",
                           "-Wno-inline-asm"],
         "qsa_prefill.hip": ["-mllvm", "-amdgpu-kernarg-preload-count=11", "-Wno-inline-asm"],
         "qsa_merge.hip": ["-mllvm", "-amdgpu-kernarg-preload-count=12"]}
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, *EXTRA.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{res.stderr}")
    # hipcc's host pass does not know the packed-fp32 feature; that warning is expected
    noise = "'-packed-fp32-ops' is not a recognized feature"
    msgs = [ln for ln in res.stderr.splitlines() if noise not in ln and ln.strip()]
    if msgs:
        sys.stderr.write("\n".join(msgs) + "\n")
    return obj


def build() -> str:
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
