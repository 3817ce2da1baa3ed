"""Build libdsa.so (the C-ABI library with its gfx950 HIP kernels) in-tree, and
libdsa_checked.so, the same sources compiled with DSA_DEVICE_CHECKS (kernels
record bad device data in a check word that dsa_device_check reports)."""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libdsa.so")
LIB_CHECKED = os.path.join(PKG, "libdsa_checked.so")
SOURCES = ["api.cpp", "indexer.hip", "topk.hip", "sparse_mla.hip", "mha_prefill.hip",
           "cache_append.hip", "bench_kernels.hip"]
# per-file code-generation options: the indexer reads its MFMA results with
# VALU right away, so they are kept in VGPRs instead of AGPRs.  The attention
# kernels take maxima of MFMA results for their softmax; compiled assuming no
# NaN values, each maximum is one v_max (or one v_max3 for three) instead of
# also quieting both operands first (about 60 VALU per 64-key tile in the
# masked multi-head loop).  Their inputs must hold no NaN: for one that does,
# the outputs are unspecified.
_NO_NANS = ["-fno-honor-nans"]
FILE_FLAGS = {"indexer.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
              "sparse_mla.hip": _NO_NANS, "mha_prefill.hip": _NO_NANS}
HEADERS = ["internal.h", "device_common.h"]
ARCH = "gfx950"

FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # no packed-fp32 VALU ops in any kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def sources():
    return [os.path.join(CSRC, s) for s in SOURCES]


def stale() -> bool:
    if not os.path.exists(LIB):
        return True
    t = os.path.getmtime(LIB)
    deps = sources() + [os.path.join(CSRC, h) for h in HEADERS] + [
        os.path.join(INCLUDE, h) for h in ("dsa.h", "dsa_bench.h")]
    return any(os.path.getmtime(d) > t for d in deps)


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc failed building libdsa.so")


def build_one(out: str, verbose: bool = False, extra=()) -> str:
    """Compile every source for gfx950 (one object each) and link `out`."""
    import tempfile
    with tempfile.TemporaryDirectory(prefix="dsa_build_") as tmpdir:
        objs = []
        for src in SOURCES:
            obj = os.path.join(tmpdir, src + ".o")
            _run(["hipcc", *FLAGS, *FILE_FLAGS.get(src, []), *extra, "-I", INCLUDE, "-I", CSRC,
                  "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj], verbose)
            objs.append(obj)
        tmp = out + ".tmp"
        _run(["hipcc", f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
        os.replace(tmp, out)
    return out


def build(verbose: bool = False, extra=()) -> str:
    """Build libdsa.so and libdsa_checked.so; returns the path of libdsa.so."""
    from concurrent.futures import ThreadPoolExecutor
    with ThreadPoolExecutor(2) as ex:
        a = ex.submit(build_one, LIB, verbose, tuple(extra))
        c = ex.submit(build_one, LIB_CHECKED, verbose, tuple(extra) + ("-DDSA_DEVICE_CHECKS=1",))
        c.result()
        return a.result()


if __name__ == "__main__":
    print(build(verbose=True))
