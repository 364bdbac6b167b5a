"""The CPU suite again, with the host code built under AddressSanitizer and
UndefinedBehaviorSanitizer: the oracle (mx_oracle.c) and the C ABI's host
sources (api.cpp: validation, device check, dispatch; layout.cpp: the host
layout converter), linked with the library's regular kernel objects.  A child
pytest loads those builds (MXFP4_LIB, MX_ORACLE_LIB) with the sanitizer
runtime preloaded; any report aborts it.  GPU code is not instrumented (the
GPU tests are not run here)."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-omit-frame-pointer", "-fno-sanitize-recover=all", "-g", "-O1"]


def _asan_runtime():
    if not shutil.which("gcc"):
        return None
    p = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    return p if os.path.isabs(p) and os.path.exists(p) else None


def _kernel_objects():
    from mxfp4_precision_amd import build
    objs = [os.path.join(build.BUILD_DIR, s + ".o") for s in build.SOURCES if s.endswith(".hip")]
    if not all(os.path.exists(o) for o in objs):
        build.build()
    return objs


@pytest.mark.skipif(_asan_runtime() is None, reason="gcc's AddressSanitizer runtime is not installed")
def test_cpu_suite_under_address_and_undefined_sanitizers(tmp_path):
    if os.environ.get("MXFP4_LIB"):
        pytest.skip("already running under a replacement library")
    rocm = "/opt/rocm"
    inc = ["-D__HIP_PLATFORM_AMD__", "-I" + rocm + "/include", "-I" + os.path.join(ROOT, "include")]
    csrc = os.path.join(ROOT, "mxfp4_precision_amd", "csrc")
    oracle_so = str(tmp_path / "liboracle_san.so")
    lib_so = str(tmp_path / "libmxfp4_san.so")
    subprocess.check_call(["gcc", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-fPIC", "-shared"]
                          + SAN + [os.path.join(ROOT, "oracle", "mx_oracle.c"), "-o", oracle_so, "-lm"])
    objs = []
    for src in ("api.cpp", "layout.cpp"):
        o = str(tmp_path / (src + ".o"))
        subprocess.check_call(["g++", "-std=c++17", "-fPIC", "-c"] + SAN + inc + [os.path.join(csrc, src), "-o", o])
        objs.append(o)
    subprocess.check_call(["g++", "-shared", "-fsanitize=address,undefined", "-o", lib_so] + objs
                          + _kernel_objects() + ["-L" + rocm + "/lib", "-lamdhip64", "-Wl,-rpath," + rocm + "/lib"])
    for so in (oracle_so, lib_so):
        syms = subprocess.run(["nm", "-D", so], capture_output=True, text=True).stdout
        assert "__asan_report" in syms and "__ubsan_handle" in syms, so
    env = dict(os.environ, LD_PRELOAD=_asan_runtime(), MXFP4_LIB=lib_so, MX_ORACLE_LIB=oracle_so,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    # the child checks that the sanitized builds are the ones it runs
    probe = ("import mxfp4_precision_amd as mx, oracle; mx.lib(); oracle.lib(); "
             "m = open('/proc/self/maps').read(); "
             "assert %r in m and %r in m and 'libasan' in m, 'sanitized builds not loaded'" % (lib_so, oracle_so))
    subprocess.check_call([sys.executable, "-c", probe], cwd=ROOT, env=env)
    r = subprocess.run([sys.executable, "-m", "pytest", "tests", "-m", "not gpu", "-x", "-q", "-p", "no:cacheprovider",
                        "--deselect", "tests/test_sanitizers.py"], cwd=ROOT, env=env, capture_output=True, text=True)
    tail = (r.stdout + r.stderr)[-3000:]
    assert r.returncode == 0, tail
    assert " passed" in tail and "ERROR: AddressSanitizer" not in tail and "runtime error" not in tail, tail
