"""Host code under AddressSanitizer + UndefinedBehaviorSanitizer (CPU only).

The fp64 oracle is built with gcc and every one of its functions is run on small ragged
shapes (tests/sanitize/oracle_driver.c).  The library's host side -- argument
validation, workspace sizing, ring set-up and the chunk-aware schedule -- is built with
the host sanitizers on (device code unchanged) and driven through the C ABI without a
GPU (tests/sanitize/abi_driver.cpp).  A report from either sanitizer fails the test."""

import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parents[1]
SAN = ROOT / "tests" / "sanitize"
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1",
           UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(map(str, cmd))}\n{r.stdout}\n{r.stderr}"
    return r


def test_oracle_under_sanitizers(tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    exe = tmp_path / "oracle_driver"
    _run(["gcc", "-std=c11", "-O1", "-g", "-fno-omit-frame-pointer", "-fopenmp", "-ffp-contract=off",
          "-fsanitize=address,undefined", "-fno-sanitize-recover=all", f"-I{ROOT / 'oracle'}",
          str(SAN / "oracle_driver.c"), str(ROOT / "oracle" / "hf_oracle.c"), "-lm", "-o", str(exe)])
    r = _run([str(exe)], env=ENV, timeout=120)
    assert "oracle driver: ok" in r.stdout


HIPCC = "/opt/rocm/bin/hipcc"
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]


@pytest.mark.timeout(600)
def test_library_host_code_under_sanitizers(tmp_path):
    if not Path(HIPCC).exists():
        pytest.skip("hipcc not available")
    from hybrid_sparse_linear_hf_amd import build as B
    csrc = B.CSRC
    flags = [f"--offload-arch={B.ARCH}", "-O1", "-g", "-std=c++17", "-fPIC", *HOST_SAN,
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]

    def compile_one(src):
        obj = tmp_path / (Path(src).stem + ".o")
        _run([HIPCC, *flags, "-c", str(csrc / src), "-o", str(obj)])
        return obj

    with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(compile_one, B.SOURCES))
    lib = tmp_path / "libhf_san.so"
    _run([HIPCC, f"--offload-arch={B.ARCH}", "-shared", "-fPIC", *HOST_SAN[:4], "-o", str(lib), *map(str, objs)])
    exe = tmp_path / "abi_driver"
    _run([HIPCC, "-O1", "-g", "-std=c++17", *HOST_SAN, f"-I{ROOT / 'include'}", str(SAN / "abi_driver.cpp"),
          f"-L{tmp_path}", "-lhf_san", f"-Wl,-rpath,{tmp_path}", "-o", str(exe)])
    r = _run([str(exe)], env=ENV, timeout=120)
    assert "abi driver: ok" in r.stdout
