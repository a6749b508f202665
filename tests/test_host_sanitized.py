"""The host side of libea under AddressSanitizer and UndefinedBehaviorSanitizer.

Builds the library's translation units with the sanitizers on the host pass
only (device code is compiled as for the product) and links them with
tests/host_checks.cpp, which drives every host path of the C ABI: sizing,
offsets, ratios, the decode-cache layout and the argument checks of every
device entry point (all rejected before any HIP call, so no GPU is used).
"""

import concurrent.futures as cf
import glob
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
CLANGXX = "/opt/rocm/llvm/bin/clang++"
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANGXX)), reason="needs hipcc")
def test_host_code_under_asan_and_ubsan(tmp_path):
    srcs = sorted(glob.glob(os.path.join(ROOT, "hybrid_sparse_full_amd", "csrc", "*.hip")))
    flags = ["-O1", "-g", "-std=c++17", "-fPIC", "--offload-arch=gfx950",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", *SAN]

    def comp(src):
        obj = str(tmp_path / (os.path.basename(src)[:-4] + ".o"))
        p = subprocess.run([HIPCC, *flags, "-c", src, "-o", obj], capture_output=True, text=True)
        assert p.returncode == 0, p.stderr[-3000:]
        return obj

    with cf.ThreadPoolExecutor(max_workers=8) as ex:
        objs = list(ex.map(comp, srcs))
    exe = str(tmp_path / "host_checks")
    p = subprocess.run([CLANGXX, "-O1", "-g", "-std=c++17", "-fsanitize=address,undefined",
                        "-fno-sanitize-recover=undefined", os.path.join(ROOT, "tests", "host_checks.cpp"),
                        *objs, "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib", "-o", exe],
                       capture_output=True, text=True)
    assert p.returncode == 0, p.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", HIP_VISIBLE_DEVICES="")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=600)
    assert r.returncode == 0, (r.stdout[-2000:], r.stderr[-4000:])
    assert "host checks passed" in r.stdout
