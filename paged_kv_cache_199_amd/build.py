"""Build libpkv.so in-tree with hipcc for gfx950 (no GPU needed: hipcc cross-compiles).

    python -m paged_kv_cache_199_amd.build
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libpkv.so")
ARCH = os.environ.get("PKV_OFFLOAD_ARCH", "gfx950")

SOURCES = ["pkv_api.hip", "kv_cache_write.hip", "decode_valu.hip", "decode_mfma.hip",
           "decode_combine.hip", "block_manager.hip", "decode_prefix.hip", "prefill_mfma.hip",
           "check_inputs.hip"]
# the benchmark's page-stream probe (include/pkv_probe.h) is a library of its own, not part of libpkv.so
PROBE_SOURCES = ["stream_probe.hip"]
PROBE_LIB = os.path.join(PKG, "libpkv_probe.so")

FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # keep the compiler from forming packed fp32 (v_pk_*_f32) instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    f"-I{os.path.join(ROOT, 'include')}",
]
# matrix-core accumulators in ordinary VGPRs (the softmax rescale then needs no AGPR copies), except
# where a wave's accumulators outgrow the VGPRs
VGPR_FORM = ["-mllvm", "-amdgpu-mfma-vgpr-form"]
AGPR_ACC: set = set()


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    return subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)


def _finish(p, verbose):
    _, stderr = p.communicate()
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in (stderr or "").splitlines() if noise not in l)
    if p.returncode != 0:
        raise RuntimeError(f"hipcc failed ({p.returncode}):\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)


def build_library(verbose: bool = False) -> str:
    """Every source to an object (in parallel), then the shared libraries: libpkv.so (the product) and
    libpkv_probe.so (the benchmark's page-stream probe)."""
    objdir = os.path.join(PKG, "_build")
    os.makedirs(objdir, exist_ok=True)
    all_src = SOURCES + PROBE_SOURCES
    jobs = max(1, min(len(all_src), int(os.environ.get("MAX_JOBS", os.cpu_count() or 4))))
    objs, pending = {}, []
    for src in all_src:
        obj = os.path.join(objdir, src.replace(".hip", ".o"))
        objs[src] = obj
        extra = [] if src in AGPR_ACC else VGPR_FORM
        pending.append([hipcc(), *FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj])
    running = []
    while pending or running:
        while pending and len(running) < jobs:
            running.append(_run(pending.pop(0), verbose))
        _finish(running.pop(0), verbose)
    for lib, srcs in ((LIB, SOURCES), (PROBE_LIB, PROBE_SOURCES)):
        tmp = lib + ".tmp"
        p = _run([hipcc(), "-shared", f"--offload-arch={ARCH}", *[objs[x] for x in srcs], "-o", tmp], verbose)
        _finish(p, verbose)
        os.replace(tmp, lib)
    return LIB


if __name__ == "__main__":
    print(build_library(verbose=True))
