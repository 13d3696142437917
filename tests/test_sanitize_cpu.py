"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

Two programs are built into a temporary folder and run:

- ``tests/sanitize/abi_host_check.cpp`` against every library source compiled
  for the host with both sanitizers (the device code objects of the regular
  build are embedded unchanged, and nothing is launched): the argument
  validation of every entry point, which must reject bad calls before any
  launch, and the host-side hybrid plan checked against its definition on
  random trees with exact-size buffers;
- ``tests/sanitize/oracle_host_check.c`` against the C oracle built with
  gcc and both sanitizers, on one thread and on four.

Leak detection is on for both; undefined behaviour aborts.
"""

import os
import shutil
import subprocess

import pytest

from linear_attention_gdn_amd import build as B

HERE = os.path.dirname(os.path.abspath(__file__))
REPO = os.path.dirname(HERE)
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
CLANGXX = os.path.join(ROCM, "llvm", "bin", "clang++")

# sanitizer flags for the host side of hipcc compiles only (the device side
# is taken from the regular build)
HOST_SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                 "-Xarch_host", "-fno-sanitize-recover=all"]
LINK_SANITIZE = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:halt_on_error=1:abort_on_error=0",
           UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout[-4000:]}\n{r.stderr[-4000:]}"
    return r


def _fatbin(src):
    stem = os.path.basename(src)
    return os.path.join(B.HERE, "_build", f"{stem}-hip-amdgcn-amd-amdhsa.hipfb")


@pytest.mark.timeout(600)
def test_abi_host_code_under_sanitizers(tmp_path):
    if not os.path.exists(B.hipcc()) or not os.path.exists(CLANGXX):
        pytest.skip("ROCm compilers not found")
    if not all(os.path.exists(_fatbin(s)) for s in B.sources()):
        B.build()
    objs = []
    for src in B.sources():
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        _run([B.hipcc(), "--offload-host-only", "-O1", "-g", "-std=c++17", "-fPIC",
              *HOST_SANITIZE, "-Xclang", "-fcuda-include-gpubinary", "-Xclang", _fatbin(src),
              "-c", src, "-o", obj])
        objs.append(obj)
    exe = str(tmp_path / "abi_host_check")
    _run([CLANGXX, "-O1", "-g", "-std=c++17", "-fno-omit-frame-pointer", *LINK_SANITIZE,
          os.path.join(HERE, "sanitize", "abi_host_check.cpp"), *objs,
          f"-L{ROCM}/lib", "-lamdhip64", f"-Wl,-rpath,{ROCM}/lib", "-o", exe])
    r = _run([exe], env=ENV, timeout=300)
    assert " 0 failed" in r.stdout


@pytest.mark.timeout(300)
def test_oracle_under_sanitizers(tmp_path):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not found")
    exe = str(tmp_path / "oracle_host_check")
    _run([gcc, "-O1", "-g", "-std=c11", "-fopenmp", "-fno-omit-frame-pointer", *LINK_SANITIZE,
          os.path.join(REPO, "oracle", "gdn_oracle.c"),
          os.path.join(HERE, "sanitize", "oracle_host_check.c"), "-o", exe, "-lm"])
    r = _run([exe], env=ENV, timeout=200)
    assert " 0 failed" in r.stdout
