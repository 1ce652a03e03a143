"""Build the sanitizer checks of the CPU tier into tests/sanitize/_build/:

* host_check: every libw4 source compiled with AddressSanitizer and
  UndefinedBehaviorSanitizer on the host side only (the device code is built as
  usual), linked with host_check.cpp;
* oracle_check: the oracle's C source and oracle_check.c, both sanitizers.

Rebuilt only when a source changed (a digest of every input is kept beside the
binaries)."""
import concurrent.futures as cf
import glob
import hashlib
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
OUT = os.path.join(HERE, "_build")
HIPCC = "/opt/rocm/bin/hipcc"
CLANGXX = "/opt/rocm/lib/llvm/bin/clang++"
SAN = ["address", "undefined"]
HOST_SAN = [f for s in SAN for f in ("-Xarch_host", f"-fsanitize={s}")] + [
    "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]


def _sources():
    return sorted(glob.glob(os.path.join(ROOT, "bit_weight_only_02_amd", "csrc", "*.hip")))


def _digest(files):
    h = hashlib.sha256()
    for f in files:
        with open(f, "rb") as fh:
            h.update(f.encode() + b"\0" + fh.read())
    return h.hexdigest()


def build():
    os.makedirs(OUT, exist_ok=True)
    inputs = (_sources() + glob.glob(os.path.join(ROOT, "bit_weight_only_02_amd", "csrc", "*.h")) +
              [os.path.join(ROOT, "include", "w4.h"), os.path.join(HERE, "host_check.cpp"),
               os.path.join(HERE, "oracle_check.c"), os.path.join(ROOT, "oracle", "w4_oracle.c"), __file__])
    dig = _digest(inputs)
    stamp = os.path.join(OUT, "digest")
    if os.path.exists(stamp) and open(stamp).read() == dig and \
            all(os.path.exists(os.path.join(OUT, b)) for b in ("host_check", "oracle_check")):
        return OUT

    def obj(src):
        o = os.path.join(OUT, os.path.basename(src) + ".o")
        subprocess.run([HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
                        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                        "-I", os.path.join(ROOT, "include"), "-c", src, "-o", o] + HOST_SAN, check=True)
        return o
    with cf.ThreadPoolExecutor(max_workers=8) as ex:
        objs = list(ex.map(obj, _sources()))
    drv = os.path.join(OUT, "host_check.o")
    subprocess.run([CLANGXX, "-O1", "-g", "-std=c++17", "-fno-omit-frame-pointer",
                    "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
                    "-I", os.path.join(ROOT, "include"), "-c", os.path.join(HERE, "host_check.cpp"), "-o", drv],
                   check=True)
    subprocess.run([CLANGXX, "-fsanitize=address,undefined", "-o", os.path.join(OUT, "host_check"), drv] + objs +
                   ["-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib"], check=True)
    subprocess.run(["gcc", "-O1", "-g", "-std=c11", "-fopenmp", "-fno-omit-frame-pointer",
                    "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
                    os.path.join(ROOT, "oracle", "w4_oracle.c"), os.path.join(HERE, "oracle_check.c"),
                    "-lm", "-o", os.path.join(OUT, "oracle_check")], check=True)
    with open(stamp, "w") as f:
        f.write(dig)
    return OUT


if __name__ == "__main__":
    print(build())
    sys.exit(0)
