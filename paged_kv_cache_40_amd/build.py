"""Build the HIP library libpagedkv.so in-tree for gfx950 with hipcc.

Usage: python -m paged_kv_cache_40_amd.build [-v]
Each .hip file under csrc/ is compiled to an object in _build/ (in parallel),
then linked into paged_kv_cache_40_amd/libpagedkv.so.  The HBM streaming-read
probe that bench.py uses for context (probe/hbm_probe.hip) becomes a separate
libpa_probe.so.
"""

from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libpagedkv.so")
PROBE_SRC = os.path.join(PKG, "probe", "hbm_probe.hip")
PROBE_LIB = os.path.join(PKG, "libpa_probe.so")
ARCH = "gfx950"

# Packed FP32 instructions are disabled: hand-written and compiler-formed
# v_pk_*_f32 are kept out of every kernel.
HIPFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    "-I", os.path.join(ROOT, "include"),
]


# Per-source extra flags.  The tile kernel keeps its MFMA accumulators in VGPRs (the
# accumulator-register form made the compiler copy all accumulators every step).
EXTRA_FLAGS = {
    "pa_tile.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
}


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines()
                    if "packed-fp32-ops" not in l and l.strip() != "")
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    if verbose and out:
        print(out)


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    cc = hipcc()
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    objs = [os.path.join(BUILD, os.path.basename(s)[:-4] + ".o") for s in srcs]
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        list(ex.map(lambda so: _run([cc, *HIPFLAGS, *EXTRA_FLAGS.get(os.path.basename(so[0]), []),
                                     "-c", so[0], "-o", so[1]], verbose),
                    zip(srcs, objs)))
    tmp = LIB + ".tmp"
    _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
    os.replace(tmp, LIB)
    # measurement aid used by bench.py (not part of the attention library)
    tmp = PROBE_LIB + ".tmp"
    _run([cc, *HIPFLAGS, "-shared", PROBE_SRC, "-o", tmp], verbose)
    os.replace(tmp, PROBE_LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
