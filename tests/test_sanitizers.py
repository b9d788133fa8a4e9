"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (no GPU).

Two drivers are built in a temporary directory and run:
  * tests/sanitize/oracle_driver.c: the FP64 oracle (gcc) on small paged
    problems covering its indexing (lengths past the capacity, ragged rows,
    small and per-head masks, per-vector scales, every storage format, split
    and merge, encoders on special values);
  * tests/sanitize/abi_driver.cpp: the library's host side (validation,
    planning, workspace sizing, error strings in api.cpp) through a
    planning-only context.  api.cpp holds no device code and is compiled for
    the host with the sanitizers (each flag follows -Xarch_host); it is linked
    with the kernel objects of the regular build.
"""
import os
import shutil
import subprocess

import pytest

from paged_gqa_attention_amd import build as B

HERE = os.path.dirname(os.path.abspath(__file__))
SAN = os.path.join(HERE, "sanitize")
ENV = dict(os.environ,
           ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:exitcode=23",
           UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1:exitcode=24")


def _run(exe, tmp):
    r = subprocess.run([exe], capture_output=True, text=True, env=ENV, cwd=tmp, timeout=300)
    assert r.returncode == 0, (r.stdout + r.stderr)[-4000:]
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr[-4000:]
    return r.stdout


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not found")
def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    subprocess.check_call(["gcc", "-std=c11", "-O1", "-g", "-fno-omit-frame-pointer",
                           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
                           os.path.join(SAN, "oracle_driver.c"), "-o", exe, "-lm", "-lpthread"])
    assert "ok" in _run(exe, str(tmp_path))


def test_library_host_side_under_asan_ubsan(tmp_path):
    hipcc = B.hipcc()
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not found")
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined"]
    inc = ["-I", os.path.join(B.ROOT, "include"), "-I", B.CSRC]
    kernels = [os.path.join(B.BUILD, os.path.splitext(s)[0] + ".o") for s in B.SOURCES
               if s.endswith(".hip")]
    if not all(os.path.exists(k) for k in kernels):
        B.build()
    objs = []
    for path, lang in ((os.path.join(B.CSRC, "api.cpp"), ["-x", "hip", "--offload-host-only"]),
                       (os.path.join(SAN, "abi_driver.cpp"), [])):
        obj = str(tmp_path / (os.path.basename(path) + ".o"))
        subprocess.check_call([hipcc] + lang + ["-c", path, "-o", obj, "-O1", "-g", "-std=c++17",
                                                "-fno-omit-frame-pointer"] + inc + san,
                              stderr=subprocess.DEVNULL)
        objs.append(obj)
    exe = str(tmp_path / "abi_driver")
    subprocess.check_call([hipcc, f"--offload-arch={B.ARCH}", "-o", exe] + objs + kernels + san,
                          stderr=subprocess.DEVNULL)
    assert "0 failures" in _run(exe, str(tmp_path))
