"""Build libfattn.so in-tree with hipcc for gfx950.

    python -m exact_tiled_attention_31_amd._build [-v]

Each HIP source is compiled to an object under ``_build/`` (in parallel),
then linked into ``libfattn.so`` next to this file.  The same sources are
also built with the device counters (FATTN_DEVICE_COUNTERS, objects under
``_build_counters/``) into ``libfattn_counters.so``, the debug library that
``fa_debug_counters`` reads.  Always rebuilds both.
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG_DIR, "csrc")
BUILD_DIR = os.path.join(PKG_DIR, "_build")
LIB_PATH = os.path.join(PKG_DIR, "libfattn.so")
COUNTERS_BUILD_DIR = os.path.join(PKG_DIR, "_build_counters")
COUNTERS_LIB_PATH = os.path.join(PKG_DIR, "libfattn_counters.so")
SOURCES = ["api.hip", "fwd_bf16.hip", "fwd_fp8.hip", "fwd_f32.hip", "bwd_bf16.hip"]
# Per-source extra flags.  The backward kernels hold more than 256 registers
# per lane; by default the compiler then gives every matrix-core result an
# AGPR and copies the score accumulators out for the VALU on every tile.
# Selecting the VGPR form keeps the scores in VGPRs and lets only the
# gradient accumulators move to AGPRs.
SOURCE_FLAGS = {"bwd_bf16.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}

ARCH = "gfx950"
# Packed fp32 VALU forms are kept out of the generated code on purpose.
HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libfattn)")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # the host pass does not know the packed-fp32 feature and says so; drop that line
    out = "\n".join(line for line in r.stdout.splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in line)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out, flush=True)


def _commands(cc, flags, build_dir):
    objs, cmds = [], []
    for src in SOURCES:
        obj = os.path.join(build_dir, os.path.splitext(src)[0] + ".o")
        objs.append(obj)
        cmds.append([cc, *flags, *SOURCE_FLAGS.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj])
    return objs, cmds


def build(verbose: bool = False, extra_flags: list[str] | None = None) -> str:
    cc = hipcc()
    flags = HIP_FLAGS + list(extra_flags or [])
    plans = [(BUILD_DIR, LIB_PATH, flags),
             (COUNTERS_BUILD_DIR, COUNTERS_LIB_PATH, flags + ["-DFATTN_DEVICE_COUNTERS"])]
    jobs = []
    for build_dir, lib_path, fl in plans:
        os.makedirs(build_dir, exist_ok=True)
        objs, cmds = _commands(cc, fl, build_dir)
        jobs.append((objs, cmds, lib_path))
    all_cmds = [c for _, cmds, _ in jobs for c in cmds]
    workers = min(len(all_cmds), max(1, min(16, os.cpu_count() or 1)))
    with concurrent.futures.ThreadPoolExecutor(workers) as ex:
        for f in [ex.submit(_run, c, verbose) for c in all_cmds]:
            f.result()
    for objs, _, lib_path in jobs:
        tmp = lib_path + ".tmp"
        _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs], verbose)
        os.replace(tmp, lib_path)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
