"""The host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

Builds the fp64 oracle (oracle/sscan_oracle.c) and the C ABI's validation and
dispatch (csrc/api.cpp) with -fsanitize=address,undefined using the host
compilers (gcc / g++; no GPU code is instrumented: api.cpp is linked with the
ordinary kernel objects of the last build), then runs the oracle pins and the
ABI tests against those builds in a child process with the sanitizer runtime
preloaded. Any report ends the child with an error."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "state_space_model_sscan_amd")
SAN = ["-fsanitize=address,undefined", "-fno-omit-frame-pointer", "-fno-sanitize-recover=all", "-g", "-O1"]


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, "%s\n%s\n%s" % (" ".join(cmd), r.stdout[-4000:], r.stderr[-4000:])
    return r


def test_oracle_and_abi_under_asan_ubsan(tmp_path):
    if not shutil.which("gcc") or not shutil.which("g++"):
        pytest.skip("host compilers missing")
    objs = os.path.join(PKG, "_build")
    kernels = sorted(os.path.join(objs, f) for f in os.listdir(objs) if f.endswith(".o") and f != "api.o") \
        if os.path.isdir(objs) else []
    if not kernels:
        pytest.skip("kernel objects not built (run __graft_entry__.build())")
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    ora = str(tmp_path / "liboracle_san.so")
    _run(["gcc", *SAN, "-fopenmp", "-fPIC", "-shared", "-ffp-contract=off", "-std=c11", "-o", ora,
          os.path.join(ROOT, "oracle", "sscan_oracle.c"), "-lm"])
    api_o = str(tmp_path / "api_san.o")
    _run(["g++", *SAN, "-fPIC", "-std=c++17", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(rocm, "include"),
          "-I", os.path.join(ROOT, "include"), "-I", os.path.join(PKG, "csrc"), "-c",
          os.path.join(PKG, "csrc", "api.cpp"), "-o", api_o])
    lib = str(tmp_path / "libsscan_san.so")
    _run(["g++", "-shared", "-fsanitize=address,undefined", "-o", lib, api_o, *kernels,
          "-L", os.path.join(rocm, "lib"), "-lamdhip64", "-Wl,-rpath," + os.path.join(rocm, "lib")])
    asan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    env = dict(os.environ)
    env.update(LD_PRELOAD=asan, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", SSCAN_SAN_ORACLE=ora, SSCAN_SAN_LIBSSCAN=lib,
               PYTHONPATH=os.pathsep.join([os.path.join(ROOT, "tests", "sanitize"), ROOT]))
    r = subprocess.run([sys.executable, "-m", "pytest", "-p", "plugin", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py"), os.path.join(ROOT, "tests", "test_abi.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    tail = (r.stdout + r.stderr)[-4000:]
    assert r.returncode == 0, tail
    assert "Sanitizer" not in r.stderr, tail
    assert " passed" in r.stdout, tail
