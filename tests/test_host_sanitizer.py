"""The library's host code (argument checks, workspace sizing) built with
AddressSanitizer and UndefinedBehaviorSanitizer and driven on the CPU with
invalid and extreme arguments (tests/host_sanitizer/driver.c).  The host
objects (api.cpp, timer.cpp) are compiled with the sanitizers for the host
pass only; the kernels' objects come from the normal build; the library and
the driver are linked with g++/gcc."""
import os
import shutil
import subprocess

import pytest

from hstu_sequential_transduction_amd import build as hb

HERE = os.path.dirname(os.path.abspath(__file__))
OUT = os.path.join(hb.BUILD, "host_sanitizer")
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]
HOST_SOURCES = ["api.cpp", "timer.cpp"]


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout[-3000:]}\n{r.stderr[-3000:]}"
    return r


@pytest.fixture(scope="module")
def driver():
    if not shutil.which("gcc") or not shutil.which("g++"):
        pytest.skip("gcc/g++ not available")
    os.makedirs(OUT, exist_ok=True)
    # kernels' objects from the normal build (build() if missing)
    objs = [os.path.join(hb.BUILD, os.path.splitext(s)[0] + ".o") for s in hb.SOURCES]
    if not all(os.path.exists(o) for o in objs):
        hb.build()
    san_objs = []
    for src in HOST_SOURCES:
        o = os.path.join(OUT, os.path.splitext(src)[0] + ".o")
        _run([hb._hipcc(), *hb.COMMON, *SAN, "-g", "-x", "hip", "-c",
              os.path.join(hb.CSRC, src), "-o", o])
        san_objs.append(o)
    kern = [o for o, s in zip(objs, hb.SOURCES) if s not in HOST_SOURCES]
    lib = os.path.join(OUT, "libhstu_san.so")
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    _run(["g++", "-shared", "-fsanitize=address,undefined", *san_objs, *kern,
          f"-L{rocm}/lib", "-lamdhip64", f"-Wl,-rpath,{rocm}/lib", "-o", lib])
    exe = os.path.join(OUT, "driver")
    _run(["gcc", "-std=c11", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
          "-I", os.path.join(os.path.dirname(HERE), "include"),
          os.path.join(HERE, "host_sanitizer", "driver.c"), lib, f"-Wl,-rpath,{OUT}",
          f"-Wl,-rpath,{rocm}/lib", "-o", exe])
    return exe


def test_host_checks_under_asan_ubsan(driver):
    env = dict(os.environ,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1",
               HIP_VISIBLE_DEVICES="")
    r = subprocess.run([driver], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0 and r.stdout.strip().endswith("ok"), \
        f"rc={r.returncode}\n{r.stdout[-3000:]}\n{r.stderr[-6000:]}"
    assert "runtime error" not in r.stderr, r.stderr[-6000:]
    assert "AddressSanitizer" not in r.stderr, r.stderr[-6000:]
