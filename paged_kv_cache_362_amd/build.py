"""Build libpagedattn.so in-tree with hipcc for gfx950.

    python -m paged_kv_cache_362_amd.build [--jobs N] [--verbose]

Every source under csrc/ is compiled to an object in _build/ (in parallel),
then linked into paged_kv_cache_362_amd/libpagedattn.so. The read-bandwidth
calibration kernels (calib/, include/pa_calib.h) the benchmark runs beside the
decode are linked into their own paged_kv_cache_362_amd/libpacalib.so. Always
rebuilds both.
"""

from __future__ import annotations

import argparse
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
CALIB = os.path.join(PKG, "calib")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libpagedattn.so")
CALIB_LIB = os.path.join(PKG, "libpacalib.so")
ARCH = "gfx950"

COMMON_FLAGS = [
    "-O3", "-std=c++17", f"--offload-arch={ARCH}", "-fPIC",
    # no packed-fp32 instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


# Per-source flags. The prefill kernel rescales its MFMA accumulators with
# VALU code; with the accumulators in AGPRs the compiler copies all of them
# to VGPRs and back on every key tile, so its MFMAs write VGPRs instead. Its
# scores are never NaN (masked scores are set to -inf by select, keys past
# the context are clamped to cached ones), so maxima need no NaN quieting.
SOURCE_FLAGS = {
    "pa_prefill.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form", "-fno-honor-nans"],
}


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found (ROCm is required to build libpagedattn.so)")
    return path


def sources(folder: str = CSRC) -> list[str]:
    return sorted(os.path.join(folder, f) for f in os.listdir(folder)
                  if f.endswith((".hip", ".cpp")))


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [hipcc(), *COMMON_FLAGS, *SOURCE_FLAGS.get(os.path.basename(src), []), "-c", src,
           "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    msgs = "\n".join(line for line in (res.stdout + res.stderr).splitlines()
                     if "packed-fp32-ops" not in line)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{msgs}")
    if verbose and msgs.strip():
        print(msgs, flush=True)
    return obj


def _link(objs: list[str], lib: str, verbose: bool) -> None:
    tmp = lib + ".tmp"
    cmd = [hipcc(), "-shared", f"--offload-arch={ARCH}", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stdout}{res.stderr}")
    os.replace(tmp, lib)


def build(jobs: int | None = None, verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    calib = sources(CALIB)
    jobs = jobs or min(len(srcs) + len(calib), max(1, (os.cpu_count() or 2)))
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), srcs + calib))
    _link(objs[:len(srcs)], LIB, verbose)
    _link(objs[len(srcs):], CALIB_LIB, verbose)
    return LIB


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--jobs", type=int, default=None)
    ap.add_argument("--verbose", action="store_true")
    a = ap.parse_args(argv)
    print(build(a.jobs, a.verbose))
    return 0


if __name__ == "__main__":
    sys.exit(main())
