"""Builds libpa.so in-tree with hipcc for gfx950.

    python -m paged_attention_kv_block_amd.build [--jobs N] [--host-only]

Every HIP source is compiled with packed-fp32 instructions disabled
(``-Xclang -target-feature -Xclang -packed-fp32-ops``); the host pass warns
that it does not know that feature, which is harmless.  ``--host-only``
builds ``libpa_host.so`` from the plain C++ part with g++ (allocator, slot
mapping, closed forms), optionally with host sanitizers.
"""
from __future__ import annotations

import argparse
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libpa.so")
HOST_LIB = os.path.join(PKG, "libpa_host.so")

HIP_SOURCES = ["pa_host.cpp", "pa_cache.hip", "pa_decode.hip", "pa_prefill.hip",
               "pa_varlen.hip", "pa_graphs.hip"]
# Per-source flags.  The prefill kernel never lets a NaN reach a max or an
# exponent (scores of keys that may be unwritten are replaced by -inf with a
# select first, and their V rows are zeroed), so it drops the NaN-quieting
# of fmaxf; the varlen kernel holds the same prefill code and a decode path
# that masks the same way.  Device code only: the host-side argument checks
# keep their NaN tests.
NO_NANS = ["-Xarch_device", "-fno-honor-nans"]
EXTRA_FLAGS = {"pa_prefill.hip": NO_NANS, "pa_varlen.hip": NO_NANS}
HOST_SOURCES = ["pa_host.cpp"]
ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build(jobs: int = 8, verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    common = ["-O3", "-std=c++17", "-fPIC", f"-I{INCLUDE}", f"-I{CSRC}", "-Wall",
              "-Wno-unused-function"]
    objs, cmds = [], []
    for src in HIP_SOURCES:
        path = os.path.join(CSRC, src)
        if not os.path.exists(path):
            continue
        obj = os.path.join(BUILD, src + ".o")
        objs.append(obj)
        if src.endswith(".hip"):
            cmd = [HIPCC, f"--offload-arch={ARCH}", "-x", "hip", "-c", path, "-o", obj,
                   "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                   "-munsafe-fp-atomics"] + common + EXTRA_FLAGS.get(src, [])
        else:
            cmd = [HIPCC, "-c", path, "-o", obj] + common
        cmds.append(cmd)
    with ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        for out in ex.map(_run, cmds):
            if verbose and out.strip():
                print(out)
    tmp = LIB + ".tmp"
    _run([HIPCC, "-shared", f"--offload-arch={ARCH}", "-o", tmp] + objs)
    os.replace(tmp, LIB)
    return LIB


def build_host(sanitize: bool = False) -> str:
    """Host-only part with g++ (no HIP): allocator, slots, closed forms."""
    os.makedirs(BUILD, exist_ok=True)
    flags = ["-O1" if sanitize else "-O2", "-g", "-std=c++17", "-fPIC", "-shared",
             f"-I{INCLUDE}", f"-I{CSRC}", "-Wall"]
    if sanitize:
        flags += ["-fsanitize=address,undefined", "-fno-omit-frame-pointer"]
    out = HOST_LIB if not sanitize else os.path.join(BUILD, "libpa_host_asan.so")
    _run(["g++"] + flags + [os.path.join(CSRC, s) for s in HOST_SOURCES] + ["-o", out])
    return out


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=8)
    ap.add_argument("--host-only", action="store_true")
    ap.add_argument("--sanitize", action="store_true")
    ap.add_argument("-v", "--verbose", action="store_true")
    a = ap.parse_args(argv)
    if a.host_only:
        print(build_host(a.sanitize))
    else:
        print(build(a.jobs, a.verbose))


if __name__ == "__main__":
    sys.exit(main())
