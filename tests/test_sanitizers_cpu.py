"""AddressSanitizer + UndefinedBehaviorSanitizer runs on the CPU of the two
pieces of host code: the oracle (every entry point on small and degenerate
inputs, and its argument errors) and the C ABI's host side (the sampler,
workspace queries, status strings and every argument error of every entry
point).  Device code is compiled as usual; only host code is instrumented.
The ABI driver runs with every GPU hidden, so no call can reach a kernel."""
import concurrent.futures as cf
import glob
import os
import shutil
import subprocess

import pytest

from conftest import ROOT

HERE = os.path.join(ROOT, "tests", "sanitize")
HIPCC = "/opt/rocm/bin/hipcc"
CLANG = "/opt/rocm/llvm/bin/clang"
SAN_ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", HIP_VISIBLE_DEVICES="-1")


def run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout[-3000:]}\n{r.stderr[-3000:]}"
    return r


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_san")
    run(["gcc", "-O1", "-g", "-std=c11", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
         "-fno-omit-frame-pointer", "-o", exe, os.path.join(HERE, "oracle_driver.c"),
         os.path.join(ROOT, "oracle", "pamm_oracle.c"), "-lm"])
    r = run([exe], env=SAN_ENV)
    assert "oracle sanitizer driver ok" in r.stdout


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)), reason="needs the ROCm toolchain")
def test_abi_host_side_under_asan_ubsan(tmp_path):
    csrc = os.path.join(ROOT, "activation_compression_pamm_amd", "csrc")
    inc = os.path.join(ROOT, "include")
    host_san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                "-Xarch_host", "-fno-omit-frame-pointer"]

    def compile_one(src):
        obj = str(tmp_path / (os.path.basename(src).split(".")[0] + ".o"))
        run([HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-Xclang", "-target-feature",
             "-Xclang", "-packed-fp32-ops", *host_san, "-I", inc, "-I", csrc, "-c", src, "-o", obj])
        return obj

    with cf.ThreadPoolExecutor(4) as ex:
        objs = list(ex.map(compile_one, sorted(glob.glob(os.path.join(csrc, "*.hip")))))
    drv = str(tmp_path / "driver.o")
    run([CLANG, "-O1", "-g", "-fsanitize=address,undefined", "-fno-omit-frame-pointer", "-I", inc, "-c",
         os.path.join(HERE, "abi_driver.c"), "-o", drv])
    exe = str(tmp_path / "abi_san")
    run([HIPCC, "--offload-arch=gfx950", "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
         "-o", exe, drv, *objs])
    r = run([exe], env=SAN_ENV)
    assert "ABI sanitizer driver ok" in r.stdout
