"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

Every source is compiled with the sanitizers on its host side only (the
device code is built as usual), linked with tests/host/abi_driver.cpp, and
run with no GPU visible.  The driver sweeps the size and split queries over
ordinary and extreme shapes (signed overflow aborts the run) and calls every
entry point with arguments that fail validation, so nothing is ever
launched."""

import concurrent.futures
import os
import shutil
import subprocess

import pytest

from paged_kv_attention_out_amd import build as pkv_build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
DRIVER = os.path.join(ROOT, "tests", "host", "abi_driver.cpp")
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]


def _hipcc():
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    return None


def _run(cmd):
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, f"{' '.join(cmd)}\n{res.stdout}\n{res.stderr}"


@pytest.mark.timeout(900)
def test_host_code_under_sanitizers(tmp_path):
    hipcc = _hipcc()
    if hipcc is None:
        pytest.skip("hipcc not available")
    flags = [f for f in pkv_build.HIP_FLAGS if f not in ("-O3",)] + ["-O1", "-g"] + SAN
    objs = []

    def compile_one(src):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        _run([hipcc, *flags, "-c", src, "-o", obj])
        return obj

    with concurrent.futures.ThreadPoolExecutor(max_workers=6) as ex:
        objs = list(ex.map(compile_one, pkv_build.sources()))
    drv = str(tmp_path / "driver.o")
    _run([hipcc, "-O1", "-g", "-std=c++17", *SAN, f"-I{os.path.join(ROOT, 'include')}",
          "-x", "c++", "-c", DRIVER, "-o", drv])
    exe = str(tmp_path / "abi_driver")
    _run([hipcc, f"--offload-arch={pkv_build.ARCH}", "-Xarch_host", "-fsanitize=address",
          "-Xarch_host", "-fsanitize=undefined", drv, *objs, "-o", exe])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1",
               HIP_VISIBLE_DEVICES="-1", ROCR_VISIBLE_DEVICES="-1")
    res = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=600)
    assert res.returncode == 0, f"{res.stdout}\n{res.stderr[-4000:]}"
    assert " 0 failed" in res.stdout, res.stdout
