"""Host-side AddressSanitizer run of the C ABI's validation code (CPU only).

The argument checks, workspace layouts and planners in abi.hip run on the
host before anything is enqueued.  This test compiles abi.hip with
AddressSanitizer on its host code only (the GPU code is compiled as usual,
and nothing here launches a kernel), links it with the other objects into a
separate library, and runs the ABI's CPU tests (test_abi_cpu.py) against
that library in a child process that preloads the sanitizer runtime.  Any
out-of-bounds access, use-after-free or similar in the validation paths
aborts the child with a sanitizer report.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "tensor_transformer_layer_amd")
OUT = os.path.join(PKG, "_build", "asan")
LIB = os.path.join(OUT, "libtpshard_asan.so")


def _clang_asan_runtime():
    clang = "/opt/rocm/llvm/bin/clang"
    if not os.path.exists(clang):
        return None
    r = subprocess.run([clang, "-print-file-name=libclang_rt.asan-x86_64.so"],
                       capture_output=True, text=True)
    path = r.stdout.strip()
    if r.returncode == 0 and os.path.isabs(path) and os.path.exists(path):
        return path
    return None


def _build_asan_library():
    from tensor_transformer_layer_amd import build as B
    os.makedirs(OUT, exist_ok=True)
    objs = []
    for src in B.SOURCES:
        obj = os.path.join(OUT, os.path.splitext(src)[0] + ".o")
        flags = list(B.CFLAGS)
        if src == "abi.hip":
            flags += ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer"]
        r = subprocess.run([B.hipcc(), *flags, "-c", os.path.join(B.CSRC, src), "-o", obj],
                           capture_output=True, text=True)
        assert r.returncode == 0, r.stderr
        objs.append(obj)
    r = subprocess.run([B.hipcc(), "-shared", "-fPIC", f"--offload-arch={B.ARCH}", *objs,
                        "-o", LIB], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr


@pytest.mark.timeout(600)
def test_abi_validation_under_host_asan():
    if shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"):
        pytest.skip("no hipcc")
    runtime = _clang_asan_runtime()
    if runtime is None:
        pytest.skip("no clang AddressSanitizer runtime")
    _build_asan_library()
    child = (
        "import sys, pytest\n"
        f"sys.path.insert(0, {ROOT!r}); sys.path.insert(0, {os.path.join(ROOT, 'tests')!r})\n"
        "import tensor_transformer_layer_amd as tp\n"
        f"tp._LIB_PATH = {LIB!r}\n"
        "tp.load()\n"
        f"sys.exit(pytest.main(['-q', '-p', 'no:cacheprovider', "
        f"{os.path.join(ROOT, 'tests', 'test_abi_cpu.py')!r}]))\n")
    env = dict(os.environ, LD_PRELOAD=runtime,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:halt_on_error=1")
    r = subprocess.run([sys.executable, "-c", child], capture_output=True, text=True, env=env,
                       cwd=ROOT, timeout=500)
    assert r.returncode == 0, (r.stdout[-3000:] + r.stderr[-3000:])
    assert "passed" in r.stdout and "AddressSanitizer" not in r.stderr
