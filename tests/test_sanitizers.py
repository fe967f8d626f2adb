"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer.

The oracle (C) and the host library (C++, linked to the recording launcher
the CPU tests use) are built with gcc/g++ -fsanitize=address,undefined -- host
code only, no HIP source is involved -- and the CPU tests of both run against
those builds in a child process (the sanitizer runtime preloaded into it).
Any out-of-bounds access, use after free, signed overflow, bad shift or
misaligned access in either aborts the child, which fails the test.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "decode_attention_quantized_append_amd", "csrc")
SAN = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
       "-fPIC", "-shared"]


@pytest.fixture(scope="module")
def san_libs(tmp_path_factory):
    d = tmp_path_factory.mktemp("sanitizers")
    oracle = str(d / "liboracle_san.so")
    nodev = str(d / "libkvq_nodev_san.so")
    subprocess.run(["gcc", *SAN, "-fopenmp", "-ffp-contract=off", "-std=c11", "-o", oracle,
                    os.path.join(ROOT, "oracle", "kvq_oracle.c"), "-lm"], check=True)
    subprocess.run(["g++", *SAN, "-std=c++17", "-Wall", "-I", os.path.join(ROOT, "include"), "-o", nodev,
                    os.path.join(CSRC, "kvq_host.cpp"), os.path.join(CSRC, "kvq_nodev.cpp")], check=True)
    return oracle, nodev


def _env(libs):
    runtime = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True,
                             check=True).stdout.strip()
    return dict(os.environ, KVQ_ORACLE_LIB=libs[0], KVQ_NODEV_LIB=libs[1], LD_PRELOAD=runtime,
                ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")


def _pytest(libs, files, *extra):
    r = subprocess.run([sys.executable, "-m", "pytest", *files, "-x", "-q", "-m", "not gpu", "-p", "no:cacheprovider",
                        *extra], cwd=ROOT, env=_env(libs), capture_output=True, text=True, timeout=900)
    assert r.returncode == 0, (r.stdout[-4000:], r.stderr[-4000:])
    return r.stdout


def test_builds_are_instrumented_and_loaded(san_libs):
    for lib in san_libs:
        syms = subprocess.run(["nm", "-D", "--undefined-only", lib], capture_output=True, text=True, check=True).stdout
        assert "__asan_report_load" in syms and "__ubsan_handle_" in syms
    code = ("import os, oracle.core as oc\n"
            "from decode_attention_quantized_append_amd import kvq\n"
            "assert oc.load()._name == os.environ['KVQ_ORACLE_LIB']\n"
            "assert kvq.load_nodev()._name == os.environ['KVQ_NODEV_LIB']\n")
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=_env(san_libs), capture_output=True, text=True,
                       timeout=300)
    assert r.returncode == 0, r.stderr[-4000:]


def test_host_logic_under_sanitizers(san_libs):
    # every host-logic test but the one that loads the HIP library itself
    _pytest(san_libs, ["tests/test_host_logic.py"], "-k", "not hip_library")


def test_oracle_under_sanitizers(san_libs):
    # the codec and attention pins (the exhaustive binary16 sweep, a minute
    # under the sanitizers, runs uninstrumented in the ordinary suite)
    _pytest(san_libs, ["tests/test_oracle_codec.py", "tests/test_oracle_attention.py"], "-k", "not every_float")
