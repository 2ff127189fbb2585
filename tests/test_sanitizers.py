"""AddressSanitizer and UndefinedBehaviorSanitizer builds of the CPU oracle and of
the host side of libtria, each driven over its entry points with valid, edge and
invalid arguments (tests/sanitize/*.c).  Host code only: the device code of the
library is compiled as usual and never launched here.  Runs without a GPU."""
import concurrent.futures as cf
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
CSRC = os.path.join(ROOT, "kv_cache_eviction_tria_amd", "csrc")
ROCM = "/opt/rocm"
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
           UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, "%s\n%s\n%s" % (" ".join(cmd), r.stdout[-4000:], r.stderr[-4000:])
    return r


def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_san")
    _run(["gcc", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
          "-fno-sanitize-recover=undefined", "-fopenmp", "-std=c99",
          os.path.join(SAN, "oracle_driver.c"), os.path.join(ROOT, "oracle", "tria_oracle.c"),
          "-o", exe, "-lm"])
    r = _run([exe], env=ENV, timeout=600)
    assert "oracle driver ok" in r.stdout


@pytest.mark.skipif(not os.path.exists(os.path.join(ROCM, "bin", "hipcc")), reason="no hipcc")
def test_library_host_code_under_asan_ubsan(tmp_path):
    hipcc = os.path.join(ROCM, "bin", "hipcc")
    srcs = sorted(f for f in os.listdir(CSRC) if f.endswith(".hip"))
    # host-side instrumentation only (each sanitizer flag applies to the host pass)
    flags = ["-O1", "-g", "-fPIC", "-std=c++17", "--offload-arch=gfx950", "-Xclang",
             "-target-feature", "-Xclang", "-packed-fp32-ops", "-I" + os.path.join(ROOT, "include"),
             "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-omit-frame-pointer"]

    def compile_one(f):
        obj = str(tmp_path / (f[:-4] + ".o"))
        _run([hipcc] + flags + ["-c", os.path.join(CSRC, f), "-o", obj])
        return obj

    with cf.ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 4)) as ex:
        objs = list(ex.map(compile_one, srcs))
    lib = str(tmp_path / "libtria_san.so")
    _run([hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", "-Xarch_host",
          "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined"] + objs + ["-o", lib])
    exe = str(tmp_path / "host_san")
    _run([os.path.join(ROCM, "bin", "amdclang"), "-O1", "-g", "-fsanitize=address",
          "-fsanitize=undefined", "-fno-sanitize-recover=undefined",
          "-I" + os.path.join(ROOT, "include"), "-I" + os.path.join(ROCM, "include"),
          "-D__HIP_PLATFORM_AMD__", os.path.join(SAN, "host_driver.c"), lib,
          "-Wl,-rpath," + str(tmp_path), "-o", exe])
    r = _run([exe], env=ENV, timeout=600)
    assert "host driver ok" in r.stdout
