"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

host.cpp (argument validation, planning, workspace sizing, the CPU packer and
RTN fit, status strings) is compiled with both sanitizers on its host side
only, linked with the library's other objects (their device code untouched)
and a driver (tests/host_asan/driver.cpp) that calls every host-side entry
point of the C ABI; no call in it reaches a device. The test fails on any
sanitizer report or failed check. It reuses the objects of the last library
build (group_wise_affine_qlinear_amd/build.py) and skips when they are
missing."""
import hashlib
import os
import shutil
import subprocess

import pytest

from group_wise_affine_qlinear_amd import build as qb

HERE = os.path.dirname(os.path.abspath(__file__))
DRIVER = os.path.join(HERE, "host_asan", "driver.cpp")
OUT_DIR = os.path.join(qb.BUILD_DIR, "asan")
SAN = ["-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer"]


def _digest(paths):
    h = hashlib.sha256()
    for p in paths:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _run(cmd):
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, f"{' '.join(cmd)}\n{res.stdout}\n{res.stderr}"


def _build():
    others = [os.path.join(qb.BUILD_DIR, os.path.splitext(s)[0] + ".o") for s in qb.SOURCES if s != "host.cpp"]
    missing = [o for o in others if not os.path.exists(o)]
    if missing:
        pytest.skip(f"library objects not built ({missing[0]}): run the library build first")
    gxx = shutil.which("g++")
    if not gxx:
        pytest.skip("g++ not available")
    host_src = os.path.join(qb.CSRC, "host.cpp")
    header = os.path.join(qb.ROOT, "include", "qlinear.h")
    key = _digest([host_src, DRIVER, header] + others)
    os.makedirs(OUT_DIR, exist_ok=True)
    exe = os.path.join(OUT_DIR, f"host_asan_{key}")
    if os.path.exists(exe):
        return exe
    host_obj = os.path.join(OUT_DIR, "host_asan.o")
    drv_obj = os.path.join(OUT_DIR, "driver_asan.o")
    # host.cpp: sanitizers on the host compilation only (each flag behind -Xarch_host)
    flags = [f for f in qb.COMMON_FLAGS if f not in ("-O3",)]
    host_san = []
    for f in SAN:
        host_san += ["-Xarch_host", f]
    _run([qb.hipcc(), "-x", "hip", *flags, "-O1", "-g", *host_san, "-c", host_src, "-o", host_obj])
    _run([gxx, "-O1", "-g", *SAN, "-I", os.path.join(qb.ROOT, "include"), "-c", DRIVER, "-o", drv_obj])
    rocm_lib = "/opt/rocm/lib"
    _run([gxx, *SAN, drv_obj, host_obj, *others, "-L", rocm_lib, "-lamdhip64", f"-Wl,-rpath,{rocm_lib}",
          "-o", exe + ".tmp"])
    os.replace(exe + ".tmp", exe)
    return exe


def test_host_code_under_asan_and_ubsan():
    exe = _build()
    env = dict(os.environ)
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    env["HIP_VISIBLE_DEVICES"] = ""  # nothing here may reach a device
    res = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    report = res.stdout + res.stderr
    assert "AddressSanitizer" not in report and "runtime error" not in report, report
    assert res.returncode == 0, report
    assert "host checks passed" in res.stdout, report
