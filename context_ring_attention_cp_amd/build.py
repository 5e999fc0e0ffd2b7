"""Build libcpattn.so in place with hipcc for gfx950.

    python -m context_ring_attention_cp_amd.build

Each source is compiled to an object in ``_build/`` (in parallel), then linked
into ``context_ring_attention_cp_amd/libcpattn.so``.
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libcpattn.so")

SOURCES = ["api.cpp", "attn_mfma.hip", "attn_f32.hip", "merge_finalize.hip", "attn_bwd.hip", "ulysses.hip", "fp8.hip", "attn_fp8.hip", "v_tiles.hip", "scratch.hip", "measure.hip"]

# Per-source extra flags.  The bf16 block kernel takes maxima of MFMA results
# and masked scores, which are never NaN: without NaN semantics the compiler
# drops the canonicalising v_max that IEEE mode puts before every max.
# Infinities keep their meaning (the masks use -inf).  The global->LDS fetch
# is inline assembly that sets M0 itself (the warning about clobbering the
# reserved M0 is expected: nothing else in that kernel uses M0).
EXTRA = {"attn_mfma.hip": ["-fno-honor-nans", "-Wno-inline-asm"], "attn_bwd.hip": ["-Wno-inline-asm"],
         "measure.hip": ["-Wno-inline-asm"],
         "attn_fp8.hip": ["-fno-honor-nans", "-Wno-inline-asm"]}

HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
COMMON = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # packed fp32 VALU ops stay off (the compiler would otherwise form them itself)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-result", "-Wno-unused-function",
    "-I", os.path.join(ROOT, "include"),
]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, src + ".o")
    cmd = [HIPCC] + COMMON + EXTRA.get(src, []) + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    errs = "\n".join(line for line in (r.stdout + r.stderr).splitlines()
                     if "packed-fp32-ops" not in line)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{errs}")
    if errs.strip():
        print(errs, file=sys.stderr)
    return obj


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build()
