"""Build libkalm.so and libkalm_debug.so (gfx950) in-tree with hipcc.

Each translation unit under csrc/ is compiled to an object in _build/ and the
objects are linked into encoder_decoder_document_amd/libkalm.so; the same
sources compiled with -DKALM_DEBUG (objects in _build/debug/) give
libkalm_debug.so, whose kernels also record every index guard that fires and
whose entry points synchronise and report it.  Packed-fp32 instruction
selection is switched off for device code (the kernels are written with plain
fp32 arithmetic and never rely on packed fp32 forms).
"""
from __future__ import annotations

import concurrent.futures
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(os.path.dirname(PKG), "_build")
LIB = os.path.join(PKG, "libkalm.so")
DEBUG_LIB = os.path.join(PKG, "libkalm_debug.so")
SOURCES = ["kalm_api.hip", "pool.hip", "rows.hip", "gemm.hip", "attn.hip", "layer.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


# Per-file flags.  attn.hip: keep MFMA accumulators in the VGPR form so the
# online-softmax rescale (a VALU multiply of the accumulator) needs no
# AGPR<->VGPR copies in the tile loop.
FILE_FLAGS = {"attn.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}


def _compile(src: str, extra, debug: bool = False) -> str:
    out_dir = os.path.join(BUILD, "debug") if debug else BUILD
    obj = os.path.join(out_dir, os.path.splitext(src)[0] + ".o")
    dbg = ["-DKALM_DEBUG"] if debug else []
    cmd = [HIPCC, *CFLAGS, *dbg, *FILE_FLAGS.get(src, []), *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    msgs = [ln for ln in r.stderr.splitlines() if "packed-fp32-ops" not in ln]
    if msgs:
        sys.stderr.write("\n".join(msgs) + "\n")
    return obj


def _link(objs, lib: str) -> None:
    tmp = lib + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, lib)


def build(verbose: bool = False, extra_flags=(), debug: bool = True) -> str:
    """Compile every HIP source and link libkalm.so (and, with debug, also
    libkalm_debug.so); returns the release library's path."""
    os.makedirs(os.path.join(BUILD, "debug"), exist_ok=True)
    extra = list(extra_flags)
    if verbose:
        extra += ["-Rpass-analysis=kernel-resource-usage"]
    jobs = [(s, False) for s in SOURCES] + ([(s, True) for s in SOURCES] if debug else [])
    with concurrent.futures.ThreadPoolExecutor(max_workers=8) as ex:
        objs = list(ex.map(lambda j: _compile(j[0], extra, j[1]), jobs))
    _link(objs[:len(SOURCES)], LIB)
    if debug:
        _link(objs[len(SOURCES):], DEBUG_LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
