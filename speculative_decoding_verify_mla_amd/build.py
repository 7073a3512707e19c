"""Build libtvmla.so (HIP, gfx950) in-tree with hipcc.

    python -m speculative_decoding_verify_mla_amd.build [-v]

Each .hip file under csrc/ compiles to an object in parallel; the objects
link into speculative_decoding_verify_mla_amd/libtvmla.so next to this file.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libtvmla.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

SOURCES = ["api.hip", "split_scalar.hip", "split_mfma.hip", "split_rows.hip", "combine.hip", "defrag.hip", "tree_mask.hip"]

# Per-file flags. The MFMA split kernel keeps its accumulators in VGPRs
# (MFMA destination/accumulator in the VGPR file) so the online-softmax
# rescale is plain vector arithmetic; the query operands then sit in AGPRs,
# which the MFMA reads directly.
FILE_FLAGS = {"split_mfma.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}

# Packed fp32 VALU ops are disabled on purpose (-packed-fp32-ops): the
# compiler would otherwise form v_pk_* fp32 instructions from float code.
CFLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = (r.stdout or "") + (r.stderr or "")
    # hipcc's host pass does not know the device-only feature; that note is harmless
    noise = "'-packed-fp32-ops' is not a recognized feature"
    out = "\n".join(line for line in out.splitlines() if noise not in line)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out, flush=True)
    return out


RESOURCE_REPORT = os.path.join(BUILD, "resource_usage.txt")


def build(verbose: bool = False, resource_usage: bool = False) -> str:
    """Compile every HIP source for gfx950 and link libtvmla.so. Returns its
    path. The compiler's per-kernel resource report (registers, LDS, scratch)
    is kept in _build/resource_usage.txt (printed with resource_usage=True)."""
    os.makedirs(BUILD, exist_ok=True)
    extra = ["-Rpass-analysis=kernel-resource-usage"]

    def one(src):
        obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
        flags = [*CFLAGS, *FILE_FLAGS.get(src, []), *extra]
        out = _run([HIPCC, *flags, "-c", os.path.join(CSRC, src), "-o", obj], verbose)
        return obj, out

    with ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        results = list(ex.map(one, SOURCES))
    report = "\n".join(line for _, out in results for line in out.splitlines() if "remark:" in line)
    with open(RESOURCE_REPORT, "w") as f:
        f.write(report + "\n")
    if resource_usage:
        print(report)
    objs = [o for o, _ in results]
    tmp = LIB + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    v = "-v" in sys.argv
    path = build(verbose=v, resource_usage="--usage" in sys.argv)
    print(path)
