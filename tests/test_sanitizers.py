"""AddressSanitizer + UndefinedBehaviorSanitizer builds of the host code (CPU
only): the C oracle with a driver that calls every entry point on small
inputs, and the library's host code (the HIP sources with host-side
instrumentation only) with a driver that runs the host-only entry points and
the argument checks that return before any HIP call. Either run aborts on an
out-of-bounds access, a use after free, a leak or undefined behaviour."""
import concurrent.futures as cf
import glob
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CLANGXX = "/opt/rocm/llvm/bin/clang++"
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd[:3])} ...\n{r.stdout[-3000:]}\n{r.stderr[-3000:]}"
    return r


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_san")
    _run(["gcc", "-std=c11", "-O1", "-g", *SAN, "-Wall", "-Wno-unknown-pragmas",
          os.path.join(HERE, "oracle_driver.c"), os.path.join(ROOT, "oracle", "oracle.c"), "-o", exe, "-lm"])
    r = _run([exe], env=ENV)
    assert "oracle driver: ok" in r.stdout


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANGXX)), reason="needs hipcc")
def test_library_host_code_under_asan_ubsan(tmp_path):
    # device code is built as usual; each sanitizer flag applies to the host pass only
    host_san = []
    for f in SAN:
        host_san += ["-Xarch_host", f]
    srcs = sorted(glob.glob(os.path.join(ROOT, "weight_quantized_moe_amd", "csrc", "*.hip")))

    def compile_one(src):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        _run([HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
              "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", *host_san,
              "-I", os.path.join(ROOT, "include"), "-c", src, "-o", obj])
        return obj

    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(compile_one, srcs))
    drv = str(tmp_path / "driver.o")
    _run([CLANGXX, "-std=c++17", "-O1", "-g", *SAN, "-I", os.path.join(ROOT, "include"), "-c",
          os.path.join(HERE, "lib_driver.cpp"), "-o", drv])
    exe = str(tmp_path / "lib_san")
    _run([CLANGXX, *SAN, drv, *objs, "-o", exe, "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib"])
    r = _run([exe], env=ENV)
    assert "library driver: ok" in r.stdout
