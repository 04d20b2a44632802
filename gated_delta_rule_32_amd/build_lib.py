"""Build libkda.so for gfx950 with hipcc (in-tree, no JIT cache).

    python -m gated_delta_rule_32_amd.build_lib        # or build() from Python

Every HIP source is compiled with packed FP32 instructions disabled
(-Xclang -target-feature -Xclang -packed-fp32-ops).

The build also checks the generated gfx950 assembly of each HIP source for
one instruction pattern: an MFMA whose accumulator input is the result of an
MFMA of a different shape issued a few instructions earlier.  The compiler
inserts no wait states there, and such a pair has produced an accumulator
that misses the first product; the kernels keep every accumulation chain to
one shape, and the build fails if that ever stops being true.
"""
from __future__ import annotations

import os
import re
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libkda.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = os.environ.get("KDA_ARCH", "gfx950")

SOURCES = [
    "kda_api.cpp",
    "kda_fwd_rowsplit.hip",
    "kda_fwd_chunk.hip",
    "kda_fwd_pipe.hip",
    "kda_bwd.hip",
    "kda_infer.hip",
    "kda_noalloc.hip",
]

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
    "-Wno-unused-result",
]


_MFMA = re.compile(r"\s*(v_mfma_\S+)\s+([va]\[\d+:\d+\]),\s*\S+,\s*\S+,\s*([va]\[\d+:\d+\])")
MIXED_CHAIN_WINDOW = 8  # instructions


def mixed_mfma_chains(asm_text: str, window: int = MIXED_CHAIN_WINDOW):
    """(line, line, shape, shape, register) for each MFMA that reads as its
    accumulator the result of an MFMA of another shape issued at most
    `window` instructions before it (branches reset the window)."""
    hits = []
    recent = []  # (line index, destination, opcode)
    for i, line in enumerate(asm_text.split("\n")):
        stripped = line.strip()
        if stripped.startswith(("s_branch", "s_cbranch", "s_barrier")) or stripped.endswith(":"):
            recent = []
            continue
        m = _MFMA.match(line)
        if not m:
            continue
        op, dst, src_c = m.groups()
        for (j, d, o) in recent:
            if d == src_c and o != op and i - j <= window:
                hits.append((j + 1, i + 1, o, op, d))
        recent = [(j, d, o) for (j, d, o) in recent if i - j < window] + [(i, dst, op)]
    return hits


def _compile(src: str) -> str:
    stem = os.path.splitext(src)[0]
    obj = os.path.join(BUILD, stem + ".o")
    cmd = [HIPCC, *FLAGS, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    if src.endswith(".hip"):
        asm = os.path.join(BUILD, stem + f"-{ARCH}.s")
        cmd = [HIPCC, *FLAGS, "-x", "hip", "--cuda-device-only", "-S", os.path.join(CSRC, src),
               "-o", asm]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc -S failed for {src}:\n{r.stderr}")
        hits = mixed_mfma_chains(open(asm).read())
        if hits:
            raise RuntimeError(f"{src}: MFMA accumulation chain mixes shapes at asm lines {hits}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
