"""Build libtq.so (HIP, gfx950) in-tree.

    python -m compressed_kv_attention_tq_amd.build_lib

Each source is compiled to an object under _build/ in parallel, then linked
into compressed_kv_attention_tq_amd/libtq.so.  Always recompiles.
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
LIB = os.path.join(PKG, "libtq.so")

# (source, object name, extra flags): the decode pass kernels are built once per
# K bit width (and blocks per head) so the slow units compile in parallel.
SOURCES = [
    ("tq_api.cpp", "tq_api", []),
    ("tq_noalloc.hip", "tq_noalloc", []),
    ("tq_stream.hip", "tq_stream", []),
    ("tq_quant.hip", "tq_quant", []),
    ("tq_decode.hip", "tq_decode", []),
    ("tq_decode.hip", "tq_decode_kb2", ["-DTQ_DECODE_KB=2"]),
    ("tq_decode.hip", "tq_decode_kb3", ["-DTQ_DECODE_KB=3"]),
    ("tq_decode.hip", "tq_decode_kb4", ["-DTQ_DECODE_KB=4"]),
] + [
    # matrix-core pass: K bits (16 = K float16) x 128-element blocks per head
    ("tq_decode_mfma.hip", f"tq_decode_mfma_kb{kb}_nb{nb}", [f"-DTQ_DECODE_KB={kb}", f"-DTQ_DECODE_NB={nb}"])
    for kb in (4, 3, 2, 16) for nb in (1, 2, 4)
]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
COMMON = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # packed fp32 vector ops are kept out of every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
    "-Wall", "-Wno-unused-function",
]


def _compile(item) -> str:
    src, name, extra = item
    obj = os.path.join(BUILD, name + ".o")
    cmd = [HIPCC, *COMMON, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 4)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    shutil.move(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build()
    sys.exit(0)
