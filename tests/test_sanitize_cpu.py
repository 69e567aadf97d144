"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only;
the device code is not instrumented):

* the oracle's C core (oracle/bflyref.c), built with gcc and driven by
  tests/san/oracle_san.c over small sizes, empty inputs and bad arguments;
* the C ABI's host layer (bfly_api.hip: argument validation, size queries,
  workspace layouts), rebuilt with the sanitizers on its host pass and
  linked with the other, uninstrumented objects of the last build, driven by
  tests/san/abi_san.c through calls that are rejected, or are pure size
  queries, before any HIP call.

Any report of either sanitizer ends its program with a non-zero status."""
import os
import shutil
import subprocess

import pytest

from learnable_butterfly_rotation_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "san")
CLANG = "/opt/rocm/llvm/bin/clang"


def run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, (" ".join(cmd), r.stdout[-4000:], r.stderr[-4000:])
    return r


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not found")
def test_oracle_core_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_san")
    run(["gcc", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
         "-fno-omit-frame-pointer", "-ffp-contract=off", os.path.join(SAN, "oracle_san.c"),
         os.path.join(ROOT, "oracle", "bflyref.c"), "-lm", "-o", exe])
    r = run([exe], env=dict(os.environ, ASAN_OPTIONS="detect_leaks=1"))
    assert "all checks passed" in r.stdout


def test_abi_host_layer_under_sanitizers(tmp_path):
    objs = [os.path.join(B.OBJ, o) for src, o, _ in B.SOURCES if src != "bfly_api.hip"]
    if not all(os.path.exists(o) for o in objs):
        pytest.skip("the library's objects are not built")
    if not (os.path.exists(B.HIPCC) and os.path.exists(CLANG)):
        pytest.skip("the ROCm compilers are not installed")
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined"]
    api = str(tmp_path / "bfly_api_san.o")
    flags = [f for f in B.FLAGS if f != "-O3"]
    run([B.HIPCC, "-O1", "-g", *flags, *san, "-Xarch_host", "-fno-sanitize-recover=all",
         "-Xarch_host", "-fno-omit-frame-pointer", "-c",
         os.path.join(B.CSRC, "bfly_api.hip"), "-o", api])
    lib = str(tmp_path / "libbfly_san.so")
    run([B.HIPCC, "-shared", "-fPIC", "--offload-arch=gfx950", *san, "-shared-libsan", api, *objs,
         "-o", lib])
    rt = os.path.dirname(run([CLANG, "-print-file-name=libclang_rt.asan-x86_64.so"]).stdout.strip())
    exe = str(tmp_path / "abi_san")
    run([CLANG + "++", "-x", "c", "-O1", "-g", "-fsanitize=address,undefined",
         "-fno-sanitize-recover=all", "-shared-libsan", "-I" + os.path.join(ROOT, "include"),
         os.path.join(SAN, "abi_san.c"), "-L" + str(tmp_path), "-lbfly_san",
         "-Wl,-rpath," + str(tmp_path), "-Wl,-rpath," + rt, "-o", exe])
    # the HIP runtime keeps allocations until exit; leaks are not this layer's to report
    r = run([exe], env=dict(os.environ, ASAN_OPTIONS="detect_leaks=0"))
    assert "all checks passed" in r.stdout
