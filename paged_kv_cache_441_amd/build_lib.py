"""Build libpagedkv.so for gfx950 with hipcc (ahead of time, in-tree).

    python -m paged_kv_cache_441_amd.build_lib [--jobs N] [--host-sanitize]

Objects go to paged_kv_cache_441_amd/_build/, the library to
paged_kv_cache_441_amd/libpagedkv.so.  Every call recompiles.  The benchmark's
read-ceiling kernels (csrc/read_ceiling.hip) go to a library of their own,
libpkv_ceiling.so, which only bench.py loads.

--host-sanitize builds libpagedkv_hostsan.so instead: the same sources with the host
side (block pool, prefix cache, argument checks, launch set-up) instrumented by
AddressSanitizer and UndefinedBehaviorSanitizer, for CPU-only tests
(tests/host_sanitizers.sh); the device code is built as usual and never runs there.
"""

from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libpagedkv.so")
SOURCES = ["pkv_api.cpp", "block_pool.cpp", "cache_write.hip", "paged_attention.hip", "paged_attention_stream.hip",
           "paged_attention_multi.hip"]
CEILING_SOURCE = "read_ceiling.hip"
CEILING_LIB = os.path.join(PKG, "libpkv_ceiling.so")
HOSTSAN_LIB = os.path.join(PKG, "libpagedkv_hostsan.so")
# each sanitizer flag applies to the host compilation only
HOST_SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                 "-Xarch_host", "-fno-sanitize-recover=undefined",
                 "-Xarch_host", "-fno-omit-frame-pointer"]
ARCH = "gfx950"

COMMON = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    # packed fp32 VALU forms stay off; scalar fp32 code only
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # matrix instructions accumulate in ordinary VGPRs: with the accumulators in AGPRs,
    # the multi-token kernels copied all of them to VGPRs and back on every tile
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-I", os.path.join(ROOT, "include"),
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (needs a ROCm install)")


def _compile(src: str, extra=(), subdir: str = "") -> str:
    obj = os.path.join(BUILD, subdir, os.path.splitext(src)[0] + ".o")
    lang = ["-x", "hip"]
    cmd = [hipcc(), *lang, *COMMON, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def _link(objs, lib: str) -> None:
    tmp = lib + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)


def build(jobs: int = 4, verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        objs = list(ex.map(_compile, SOURCES + [CEILING_SOURCE]))
    _link(objs[:-1], LIB)
    _link(objs[-1:], CEILING_LIB)
    if verbose:
        print(f"built {LIB} and {CEILING_LIB}")
    return LIB


def build_host_sanitized(jobs: int = 4, verbose: bool = False) -> str:
    """libpagedkv_hostsan.so: host code under ASan + UBSan.  A shared library does not
    carry the sanitizer runtime; the process that loads it preloads the ASan runtime
    (which holds the UBSan handlers too)."""
    os.makedirs(os.path.join(BUILD, "hostsan"), exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        objs = list(ex.map(lambda src: _compile(src, HOST_SANITIZE, "hostsan"), SOURCES))
    _link(objs, HOSTSAN_LIB)
    if verbose:
        print(f"built {HOSTSAN_LIB}")
    return HOSTSAN_LIB


def main(argv=None) -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=min(8, os.cpu_count() or 1))
    ap.add_argument("--host-sanitize", action="store_true")
    args = ap.parse_args(argv)
    if args.host_sanitize:
        build_host_sanitized(args.jobs, verbose=True)
    else:
        build(args.jobs, verbose=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
