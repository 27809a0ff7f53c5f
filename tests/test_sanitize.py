"""CPU sanitizer runs: the fp64 oracle and the library's host-side argument
validation built with AddressSanitizer + UndefinedBehaviorSanitizer (host
code only, with gcc/g++; no GPU code is instrumented) and driven over every
entry point, edge shapes included.  A sanitizer report fails the run."""
import glob
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
CSRC = os.path.join(ROOT, "dependent_position_encoding_amd", "csrc")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"
    return r


def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_san")
    _run(["gcc", "-std=c11", "-O1", "-g", *SAN, "-Wall", "-Wno-unknown-pragmas", "-o", exe,
          os.path.join(HERE, "oracle_driver.c"), os.path.join(ROOT, "oracle", "path_oracle.c"),
          "-lm"])
    r = _run([exe], env={**os.environ, "ASAN_OPTIONS": "detect_leaks=1"})
    assert "ok" in r.stdout


def _kernel_objects():
    """The library's kernel objects (compiled by the in-tree build)."""
    objs = sorted(glob.glob(os.path.join(ROOT, "_build", "*.hip.o")))
    if len(objs) < len(glob.glob(os.path.join(CSRC, "*.hip"))):
        from dependent_position_encoding_amd import _build
        _build.build()
        objs = sorted(glob.glob(os.path.join(ROOT, "_build", "*.hip.o")))
    return objs


@pytest.mark.skipif(not os.path.exists("/opt/rocm/lib/libamdhip64.so"), reason="no HIP runtime")
def test_host_validation_under_asan_ubsan(tmp_path):
    inc = ["-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", "-I", os.path.join(ROOT, "include"),
           "-I", CSRC]
    host = str(tmp_path / "host_san.o")
    drv = str(tmp_path / "drv_san.o")
    _run(["g++", "-std=c++17", "-O1", "-g", *SAN, "-Wno-unused-result", *inc, "-c",
          os.path.join(CSRC, "host.cpp"), "-o", host])
    _run(["g++", "-std=c++17", "-O1", "-g", *SAN, *inc, "-c",
          os.path.join(HERE, "abi_driver.cpp"), "-o", drv])
    exe = str(tmp_path / "abi_san")
    _run(["g++", *SAN, "-o", exe, drv, host, *_kernel_objects(), "-L/opt/rocm/lib", "-lamdhip64",
          "-Wl,-rpath,/opt/rocm/lib"])
    # the HIP runtime keeps process-lifetime allocations: leak checking is off here
    r = _run([exe], env={**os.environ, "ASAN_OPTIONS": "detect_leaks=0"})
    assert "ok" in r.stdout
