"""AddressSanitizer and UndefinedBehaviorSanitizer on the CPU side:

* the oracle (plain C) built with both sanitizers and driven through every
  function and edge case (tests/sanitize/oracle_driver.c);
* the library's host code -- validation, workspace layouts and views, every
  entry point's argument checks -- built with host-only sanitizers (the
  device code is compiled as usual) and driven through its refusals with
  fake device pointers (tests/sanitize/host_driver.cpp).

A report from either sanitizer aborts its driver.  Nothing here needs or
touches a GPU."""
import os
import shutil
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CLANGXX = "/opt/rocm/llvm/bin/clang++"
CSRC = os.path.join(ROOT, "hashed_gram_embedding_amd", "csrc")
SAN = os.path.join(ROOT, "tests", "sanitize")
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
           UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", OMP_NUM_THREADS="2")


@pytest.fixture(scope="module")
def tmp():
    d = tempfile.mkdtemp(prefix="ngram_san_")
    yield d
    shutil.rmtree(d, ignore_errors=True)


def test_oracle_under_address_and_ub_sanitizers(tmp):
    exe = os.path.join(tmp, "oracle_driver")
    subprocess.run(["gcc", "-O1", "-g", "-std=c11", "-fopenmp", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=all", os.path.join(SAN, "oracle_driver.c"),
                    os.path.join(ROOT, "oracle", "ngram_oracle.c"), "-o", exe, "-lm"],
                   check=True, capture_output=True, text=True)
    r = subprocess.run([exe], capture_output=True, text=True, env=ENV, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "ran clean" in r.stdout


@pytest.mark.skipif(not os.path.exists(CLANGXX), reason="ROCm clang not installed")
def test_library_host_code_under_address_and_ub_sanitizers(tmp):
    objs, procs = [], []
    for src in sorted(os.listdir(CSRC)):
        if not src.endswith(".hip"):
            continue
        obj = os.path.join(tmp, src[:-4] + ".o")
        objs.append(obj)
        cmd = [HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
               "-I" + os.path.join(ROOT, "include"), "-I" + CSRC,
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               # host code only: each sanitizer flag is preceded by -Xarch_host
               "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
               "-Xarch_host", "-fno-sanitize-recover=all",
               "-c", os.path.join(CSRC, src), "-o", obj]
        procs.append((cmd, subprocess.Popen(cmd, stdout=subprocess.PIPE,
                                            stderr=subprocess.STDOUT, text=True)))
    for cmd, p in procs:
        out, _ = p.communicate()
        assert p.returncode == 0, " ".join(cmd) + "\n" + out
    lib = os.path.join(tmp, "libngram_san.so")
    subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC",
                    "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                    *objs, "-o", lib], check=True, capture_output=True, text=True)
    exe = os.path.join(tmp, "host_driver")
    subprocess.run([CLANGXX, "-O1", "-g", "-std=c++17", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=all", "-I" + os.path.join(ROOT, "include"),
                    os.path.join(SAN, "host_driver.cpp"), "-L" + tmp, "-lngram_san",
                    "-Wl,-rpath," + tmp, "-Wl,-rpath,/opt/rocm/lib", "-o", exe],
                   check=True, capture_output=True, text=True)
    r = subprocess.run([exe], capture_output=True, text=True, env=ENV, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "ran clean" in r.stdout
