"""Build libsinkattn.so (HIP kernels + C ABI) for gfx950, in-tree.

    python -m attention_sink_softmax_amd.build

Each source is compiled with hipcc in parallel, then linked into
attention_sink_softmax_amd/libsinkattn.so.  Objects go to attention_sink_softmax_amd/_build/.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libsinkattn.so")
SOURCES = ("api.hip", "prefill.hip", "decode.hip", "prologue.hip", "backward.hip")
# Per-source flags.  The prefill kernels never test for NaN (masked scores are -inf), so
# max/min need no NaN canonicalisation of the MFMA results; their matrix products write
# ordinary VGPRs (the softmax reads the scores with no copy out of accumulator registers,
# and the sliding-window ring kernel fits two waves per SIMD without spilling).
EXTRA = {"prefill.hip": ["-fno-honor-nans", "-mllvm", "-amdgpu-mfma-vgpr-form"]}
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-I", INCLUDE, "-I", CSRC,
    # packed fp32 VALU ops (v_pk_*_f32) are kept out of the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "is not a recognized feature" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    objs = [os.path.join(BUILD_DIR, s.rsplit(".", 1)[0] + ".o") for s in SOURCES]
    cmds = [[HIPCC, *FLAGS, *EXTRA.get(s, []), "-c", os.path.join(CSRC, s), "-o", o] for s, o in zip(SOURCES, objs)]
    with ThreadPoolExecutor(len(cmds)) as ex:
        outs = list(ex.map(_run, cmds))
    tmp = LIB + ".tmp"
    outs.append(_run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]))
    os.replace(tmp, LIB)
    if verbose:
        for o in outs:
            if o.strip():
                print(o)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
