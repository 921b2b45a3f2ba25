"""Build libplora.so in-tree for gfx950 (hipcc) -- no JIT, no torch extension.

    python packed_adapter_lora_amd/build.py

Every HIP source is compiled with packed-fp32 instructions disabled (the
compiler otherwise forms v_pk_* fp32 ops from ordinary float code).
"""
from __future__ import annotations

import glob
import hashlib
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libplora.so")
ARCH = "gfx950"

HIP_SOURCES = ["api.hip", "api_noalloc.hip", "api_block.hip", "gemm_bf16.hip", "lora_bf16.hip", "kernels_f32.hip", "optim.hip",
               "block.hip", "attention.hip", "attention_dkv.hip", "probes.hip"]
CXX_SOURCES = ["plan.cpp", "planner.cpp"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
HIP_FLAGS = ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-Wall",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-I", INCLUDE, "-I", CSRC]
CXX_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-I", INCLUDE, "-I", CSRC]
# Per-source extra flags.  The attention kernels keep their matrix-core
# accumulators in ordinary VGPRs: left to its heuristics the compiler places
# the dK/dV accumulators in AGPRs and copies them to and from VGPRs around
# every query tile.
EXTRA_FLAGS = {"attention.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
               "attention_dkv.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def source_hash() -> str:
    """16 hex digits over the library's sources, headers and compile flags
    (paths relative to the repository, so the same tree hashes the same on
    any machine).  The library carries the hash it was built from
    (plora_source_hash), and the package refuses a library whose hash differs
    from the sources beside it."""
    h = hashlib.sha256()
    files = sorted(glob.glob(os.path.join(CSRC, "*")) + glob.glob(os.path.join(INCLUDE, "*.h")))
    for f in files:
        if not os.path.isfile(f):
            continue
        h.update(os.path.relpath(f, ROOT).encode() + b"\0")
        with open(f, "rb") as fh:
            h.update(fh.read())
    flags = [x.replace(ROOT, ".") for x in HIP_FLAGS + CXX_FLAGS] + sorted(
        k + ":" + " ".join(v) for k, v in EXTRA_FLAGS.items())
    h.update("\0".join(flags).encode())
    return h.hexdigest()[:16]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # the host pass of hipcc does not know the packed-fp32 feature; that note is harmless
    out = "\n".join(ln for ln in r.stdout.splitlines() if "packed-fp32-ops" not in ln)
    if r.returncode != 0:
        raise RuntimeError("build failed: %s\n%s" % (" ".join(cmd), out))
    return out


def build(verbose: bool = False, jobs: int = 8) -> str:
    os.makedirs(BUILD, exist_ok=True)
    stamp = ["-DPLORA_SOURCE_HASH=\"%s\"" % source_hash()]
    jobs_list = []
    for s in HIP_SOURCES:
        obj = os.path.join(BUILD, s + ".o")
        extra = EXTRA_FLAGS.get(s, []) + (stamp if s == "api.hip" else [])
        jobs_list.append([HIPCC] + HIP_FLAGS + extra + ["-c", os.path.join(CSRC, s), "-o", obj])
    for s in CXX_SOURCES:
        obj = os.path.join(BUILD, s + ".o")
        jobs_list.append(["g++"] + CXX_FLAGS + ["-c", os.path.join(CSRC, s), "-o", obj])
    with ThreadPoolExecutor(max_workers=max(1, min(jobs, len(jobs_list)))) as ex:
        outs = list(ex.map(_run, jobs_list))
    if verbose:
        for o in outs:
            if o.strip():
                print(o)
    objs = [os.path.join(BUILD, s + ".o") for s in HIP_SOURCES + CXX_SOURCES]
    tmp = LIB + ".tmp%d" % os.getpid()
    _run([HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
