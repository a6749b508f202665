"""Build libea.so (HIP, gfx950) in-tree.

    python -m hybrid_sparse_full_amd.build [--jobs N]

Compiles every csrc/*.hip translation unit with hipcc for gfx950 and links
them into hybrid_sparse_full_amd/libea.so.  Packed fp32 vector instructions
are disabled on the device side (-packed-fp32-ops); the host pass warns that
it does not know that target feature, which is harmless.
"""

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
OBJ = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libea.so")
ARCH = os.environ.get("EA_OFFLOAD_ARCH", "gfx950")

HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
CFLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _compile(src):
    obj = os.path.join(OBJ, os.path.basename(src)[:-4] + ".o")
    cmd = [HIPCC, *CFLAGS, "-c", src, "-o", obj]
    p = subprocess.run(cmd, capture_output=True, text=True)
    warn = "\n".join(l for l in (p.stderr or "").splitlines()
                     if "packed-fp32-ops" not in l)
    return src, obj, p.returncode, warn


def build(jobs=None, verbose=False):
    os.makedirs(OBJ, exist_ok=True)
    srcs = sources()
    objs = []
    with cf.ThreadPoolExecutor(max_workers=jobs or min(8, len(srcs))) as ex:
        for src, obj, rc, warn in ex.map(_compile, srcs):
            if warn.strip() and (verbose or rc):
                print(warn, file=sys.stderr)
            if rc:
                raise RuntimeError(f"hipcc failed on {os.path.basename(src)}")
            objs.append(obj)
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    p = subprocess.run(cmd, capture_output=True, text=True)
    if p.returncode:
        print(p.stderr, file=sys.stderr)
        raise RuntimeError("link of libea.so failed")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=None)
    ap.add_argument("-v", "--verbose", action="store_true")
    a = ap.parse_args()
    print(build(a.jobs, a.verbose))
