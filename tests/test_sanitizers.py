"""The library's host-side checks (gdn_api.cpp: geometry validation,
workspace sizing, argument refusals) built with AddressSanitizer and
UndefinedBehaviorSanitizer and driven through every refusal path by a C
program (tests/abi_refusals.c).  CPU only: no call passes validation, so no
kernel is launched; the HIP objects are the library's normal build."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "gated_deltanet_delta_amd", "csrc")
BUILD = os.path.join(ROOT, "_build")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]


def _hip_objects():
    objs = [os.path.join(BUILD, n + ".o") for n in ("gdn_step.hip", "gdn_prefill.hip")]
    if not all(os.path.exists(o) for o in objs):
        from gated_deltanet_delta_amd import build
        build.build()
    return objs


def test_host_checks_clean_under_asan_and_ubsan(tmp_path):
    if shutil.which("g++") is None or shutil.which("gcc") is None:
        pytest.skip("no host compiler")
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]
    api = str(tmp_path / "api.o")
    drv = str(tmp_path / "drv.o")
    exe = str(tmp_path / "abi_refusals")
    subprocess.run(["g++", "-std=c++17", "-fPIC", *SAN, *inc, "-D__HIP_PLATFORM_AMD__",
                    "-I", os.path.join(rocm, "include"), "-c", os.path.join(CSRC, "gdn_api.cpp"), "-o", api],
                   check=True)
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", *SAN, *inc,
                    "-c", os.path.join(ROOT, "tests", "abi_refusals.c"), "-o", drv], check=True)
    subprocess.run(["g++", *SAN, drv, api, *_hip_objects(), "-L", os.path.join(rocm, "lib"), "-lamdhip64",
                    "-Wl,-rpath," + os.path.join(rocm, "lib"), "-o", exe], check=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0, (r.returncode, r.stdout, r.stderr[-4000:])
    assert "abi refusals ok" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr[-4000:]
