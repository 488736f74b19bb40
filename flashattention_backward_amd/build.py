"""Build libfab.so in-tree with hipcc for gfx950 (no GPU needed: hipcc cross-compiles).

    python -m flashattention_backward_amd.build        # or __graft_entry__.build()

Each .hip source is compiled to an object under ``_build/`` in parallel, then linked into
``flashattention_backward_amd/libfab.so``.  Always recompiles (the build check must exercise the
compiler every time).
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libfab.so")
SOURCES = ["api.hip", "preprocess.hip", "bwd_dkdv.hip", "bwd_dq.hip", "bwd16.hip", "fwd.hip", "fwd16.hip"]

HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")
# Packed-fp32 VALU forms are disabled for all device code (see the design notes).
DEVICE_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
                "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                "-Wno-unused-command-line-argument"]


# Per-source extra flags.  bwd16.hip keeps its long-lived accumulators in AGPRs through
# inline-asm MFMAs; every other MFMA there is selected in VGPR form so that the short-lived
# score tiles never compete with the accumulators for AGPRs.
EXTRA_FLAGS = {"bwd16.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
               "fwd16.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


# Sources with inline-asm MFMAs: compiled with -save-temps so that the device assembly of the
# very object that is linked can be checked for operand hazards (asm_check).
ASM_CHECKED = {"bwd16.hip"}


def device_asm_path(src: str) -> str:
    stem = os.path.splitext(src)[0]
    return os.path.join(BUILD, stem + "_temps", f"{stem}-hip-amdgcn-amd-amdhsa-gfx950.s")


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0].replace("/", "_") + ".o")
    cmd = [HIPCC, *DEVICE_FLAGS, *EXTRA_FLAGS.get(src, []), "-I", os.path.join(ROOT, "include"),
           "-c", os.path.join(CSRC, src), "-o", obj]
    cwd = None
    if src in ASM_CHECKED:
        cwd = os.path.dirname(device_asm_path(src))
        os.makedirs(cwd, exist_ok=True)
        cmd.append("-save-temps")
    r = subprocess.run(cmd, capture_output=True, text=True, cwd=cwd)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    if src in ASM_CHECKED:
        from . import asm_check
        with open(device_asm_path(src)) as fh:
            asm = fh.read()
        bad = asm_check.mfma_operand_hazards(asm)
        if bad:
            lines = "\n".join(f"  {p}  ->  {m}" for p, m in bad[:10])
            raise RuntimeError(f"{src}: {len(bad)} MFMA operand hazard(s) in the compiled code:\n{lines}")
    return obj


def _link(objs, out: str):
    tmp = out + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, out)


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    _link(objs, LIB)
    if verbose:
        print(f"[fab] built {LIB}")
    return LIB


if __name__ == "__main__":
    build()
    sys.exit(0)
