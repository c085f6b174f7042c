"""Host-side sanitizer run: the C ABI's host layer (planner, validation, size
queries) built with AddressSanitizer and UndefinedBehaviorSanitizer on the
host code only, driven by an argument fuzzer (tests/host_fuzz.cpp).  The
device code is linked unchanged from the regular build; no GPU is used."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "newton_schulz_gram_amd", "csrc")
OBJS = os.path.join(ROOT, "newton_schulz_gram_amd", "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CLANG = "/opt/rocm/llvm/bin/clang++"
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]


def _run(cmd, **kw):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, **kw)
    assert r.returncode == 0, " ".join(cmd) + "\n" + r.stdout[-4000:]
    return r.stdout


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)), reason="ROCm compilers not found")
def test_host_layer_under_asan_ubsan(tmp_path):
    kernels = [os.path.join(OBJS, f + ".o") for f in ("nsg_kernels.hip", "nsg_select.hip", "nsg_muon.hip")]
    if not all(os.path.exists(k) for k in kernels):
        pytest.skip("device objects not built (run __graft_entry__.build() first)")
    api = str(tmp_path / "nsg_api_san.o")
    _run([HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", *HOST_SAN,
          "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-x", "hip", "-c", os.path.join(CSRC, "nsg_api.cpp"),
          "-o", api])
    lib = str(tmp_path / "libnsg_san.so")
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *HOST_SAN, api, *kernels, "-o", lib])
    exe = str(tmp_path / "host_fuzz")
    _run([CLANG, "-O1", "-g", "-std=c++17", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
          "-fno-omit-frame-pointer", "-I", os.path.join(ROOT, "include"), os.path.join(ROOT, "tests", "host_fuzz.cpp"),
          lib, "-Wl,-rpath," + str(tmp_path), "-o", exe])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1", UBSAN_OPTIONS="print_stacktrace=1")
    out = _run([exe, "20000"], env=env, timeout=600)
    assert "ok 20000 iterations" in out
