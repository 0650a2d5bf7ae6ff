"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer
(CPU only).

bsa_api.cpp (argument validation, workspace carving, dispatch) is compiled
with the host sanitizers -- the device code is left as it is -- and linked
with the kernel objects into a separate library.  test_abi.py then runs in a
child process against that library, with the sanitizer runtime preloaded; a
memory error or undefined behaviour in the host code aborts the child.
The child imports only the ctypes binding (not torch).
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "block_sparse_attention_16_amd")
OUT = os.path.join(ROOT, "_build", "asan")
SAN = "-Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined".split()

RUNNER = """
import ctypes, sys, types
m = types.ModuleType("block_sparse_attention_16_amd")
m.__path__ = [{pkg!r}]
sys.modules["block_sparse_attention_16_amd"] = m
sys.path.insert(0, {root!r})
assert hasattr(ctypes.CDLL(None), "__asan_init"), "sanitizer runtime not loaded"
from block_sparse_attention_16_amd import _lib
_lib.LIB_PATH = {lib!r}
import pytest
sys.exit(pytest.main([{tests!r}, "-q", "-p", "no:cacheprovider"]))
"""


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"
    return r


def test_abi_suite_under_host_sanitizers(tmp_path):
    from block_sparse_attention_16_amd import build as B
    try:
        hipcc = B.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    B.build(verbose=False)                                     # kernel objects in _build/
    os.makedirs(OUT, exist_ok=True)
    api_obj = os.path.join(OUT, "bsa_api.o")
    flags = [f for f in B.COMMON if f != "-O3"] + ["-O1", "-g", "-fno-omit-frame-pointer"]
    _run([hipcc, "-x", "hip", *flags, *SAN, "-c", os.path.join(B.CSRC, "bsa_api.cpp"), "-o", api_obj])
    kernels = [os.path.join(B.BUILD, os.path.splitext(s)[0] + ".o") for s in B.SOURCES if s != "bsa_api.cpp"]
    lib = os.path.join(OUT, "libbsa_asan.so")
    _run([hipcc, f"--offload-arch={B.ARCH}", "-shared", "-fPIC", "-shared-libsan", *SAN, "-o", lib, *kernels,
          api_obj])
    rt = _run([hipcc, "-print-file-name=libclang_rt.asan-x86_64.so"]).stdout.strip()
    if not os.path.isabs(rt) or not os.path.exists(rt):
        pytest.skip("sanitizer runtime not found")
    script = tmp_path / "run_abi.py"
    script.write_text(RUNNER.format(pkg=PKG, root=ROOT, lib=lib, tests=os.path.join(ROOT, "tests", "test_abi.py")))
    env = dict(os.environ, LD_PRELOAD=rt, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, str(script)], capture_output=True, text=True, env=env, timeout=600)
    assert r.returncode == 0, f"ABI tests under sanitizers failed:\n{r.stdout[-4000:]}\n{r.stderr[-4000:]}"
    assert "passed" in r.stdout and "failed" not in r.stdout, r.stdout[-2000:]
