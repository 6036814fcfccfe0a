"""Build libsmla.so (HIP, gfx950) in-tree with hipcc, and libsmla_peak.so (the achievable-peak
microbenchmarks of csrc/peak.hip, measurement only).

    python -m sparse_mla_decode_topk_amd.build

Each source is compiled to its own object (in parallel), then the objects are linked.  The
fp8_ds_mla decode is compiled with the compiler's MFMA register form pinned to VGPRs: its score
MFMAs accumulate in VGPRs that the vector unit reads, while its output MFMAs, written as inline
assembly, keep their accumulators in the AGPRs.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libsmla.so")
PEAK_LIB = os.path.join(PKG, "libsmla_peak.so")
SOURCES = ["smla_api.hip", "convert_index.hip", "decode_row.hip", "merge_lse.hip", "cache_write.hip", "dense_slots.hip",
           "decode_bf16.hip", "split_combine.hip"]
EXTRA_FLAGS = {"decode_row.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}
ARCH = os.environ.get("SMLA_OFFLOAD_ARCH", "gfx950")
COMMON = ["-O3", "-std=c++17", "-fPIC",
          # keep packed-fp32 VALU instructions (v_pk_*_f32) out of the generated code
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _run(cmd):
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + " ".join(cmd) + "\n" + res.stdout + res.stderr)
    return res.stdout


def build(verbose: bool = False) -> str:
    """Compile every HIP source and link LIB and PEAK_LIB; returns LIB's path."""
    cc = hipcc()
    with tempfile.TemporaryDirectory(prefix="smla_build_") as tmp:
        def compile_one(src):
            obj = os.path.join(tmp, os.path.splitext(src)[0] + ".o")
            _run([cc, f"--offload-arch={ARCH}", *COMMON, *EXTRA_FLAGS.get(src, []), "-I", os.path.join(ROOT, "include"),
                  "-c", os.path.join(CSRC, src), "-o", obj])
            return obj

        with ThreadPoolExecutor(max_workers=min(8, len(SOURCES) + 1)) as ex:
            objs = list(ex.map(compile_one, SOURCES + ["peak.hip"]))
        for lib, group in ((LIB, objs[:-1]), (PEAK_LIB, objs[-1:])):
            out = lib + ".tmp"
            log = _run([cc, f"--offload-arch={ARCH}", "-fPIC", "-shared", "-o", out, *group])
            if verbose:
                sys.stdout.write(log)
            os.replace(out, lib)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
