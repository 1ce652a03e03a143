"""Build libw4.so (the HIP library) in-tree with hipcc for gfx950.

Every source compiles to its own object (in parallel), then one link step makes
the shared library.  Each translation unit holds its kernels together with the
host code that launches them, so no relocatable device code is needed.
"""

from __future__ import annotations

import glob
import os
import subprocess
import tempfile
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libw4.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Wall", "-Wno-unused-function",
    # no packed-fp32 VALU instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def sources():
    return sorted(glob.glob(os.path.join(HERE, "csrc", "*.hip")))


def build(verbose: bool = False, jobs: int | None = None) -> str:
    """Compile every HIP source into bit_weight_only_02_amd/libw4.so."""
    srcs = sources()
    jobs = jobs or min(len(srcs), max(1, min(16, os.cpu_count() or 1)))
    with tempfile.TemporaryDirectory(prefix="w4build_") as tmpdir:
        objs = [os.path.join(tmpdir, os.path.basename(s) + ".o") for s in srcs]

        def compile_one(pair):
            src, obj = pair
            cmd = [HIPCC, *FLAGS, "-c", "-o", obj, src]
            if verbose:
                print(" ".join(cmd), flush=True)
            r = subprocess.run(cmd, capture_output=True, text=True)
            return src, r

        with ThreadPoolExecutor(max_workers=jobs) as ex:
            results = list(ex.map(compile_one, zip(srcs, objs)))
        failed = [(s, r) for s, r in results if r.returncode != 0]
        for s, r in results:
            # warnings other than the host pass's note on the packed-fp32 feature
            lines = [ln for ln in (r.stderr or "").splitlines() if "packed-fp32-ops" not in ln]
            if lines and (verbose or r.returncode != 0):
                print("\n".join(lines), flush=True)
        if failed:
            raise subprocess.CalledProcessError(failed[0][1].returncode, failed[0][0])
        tmp = LIB + ".tmp"
        cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.check_call(cmd)
        os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
