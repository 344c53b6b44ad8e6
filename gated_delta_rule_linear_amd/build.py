"""Build ``liblinattn.so`` (HIP, gfx950) in-tree.

Every translation unit under ``csrc/`` is compiled with hipcc for gfx950 and
linked into one shared library next to this file. Usage:
``python -m gated_delta_rule_linear_amd.build [-j N]``.
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "liblinattn.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

COMMON = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-Wno-unused-function", "-Wno-unused-variable",
    # packed fp32 ops disabled for all device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]

SOURCES = ["la_api.cpp", "decode.hip", "prefill_valu.hip", "prefill_kath_mfma.hip", "prefill_kda_mfma.hip",
           "selective_scan.hip", "backward_valu.hip", "backward_gdn_valu.hip", "backward_ssd_mfma.hip",
           "backward_gdn_mfma.hip",
           "prefill_gla_mfma.hip", "prefill_gdn_mfma.hip", "noalloc.hip", "stream_rmw.hip",
           "prefill_ssd_mfma.hip"]


# per-file code generation options: matrix-core results kept in ordinary vector registers
# (no copies out of the accumulation registers) where a kernel's vector-ALU work consumes
# them every chunk
EXTRA = {"prefill_gdn_mfma.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
         "prefill_gla_mfma.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
         "prefill_kda_mfma.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC, *COMMON, *EXTRA.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    warn = "\n".join(line for line in r.stderr.splitlines()
                     if "packed-fp32-ops" not in line and line.strip())
    if warn:
        print(f"[{src}]\n{warn}")
    return obj


def build(jobs: int = 8) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("-j", type=int, default=8)
    print(build(ap.parse_args().j))
