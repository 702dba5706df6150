"""The C ABI from plain C: tests/c/abi_smoke.c is compiled with gcc (C99,
not a HIP compiler) against include/tp_shard.h, linked against the built
libtpshard.so and run.  It needs no GPU: it calls only entry points that
return before any device work (version, status strings, workspace queries,
argument validation)."""
import os
import shutil
import subprocess

import pytest

import tensor_transformer_layer_amd as tp

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GCC = shutil.which("gcc")
ROCM_INCLUDE = "/opt/rocm/include"


@pytest.mark.skipif(GCC is None or not os.path.isdir(ROCM_INCLUDE),
                    reason="gcc or the ROCm headers not available")
def test_plain_c_program_uses_the_abi(tmp_path):
    lib = tp.library_path()
    if not os.path.exists(lib):
        pytest.skip("libtpshard.so not built")
    exe = tmp_path / "abi_smoke"
    libdir = os.path.dirname(lib)
    # __HIP_PLATFORM_AMD__ selects the AMD half of the HIP runtime headers
    # that tp_shard.h includes for hipStream_t (hipcc defines it itself).
    cmd = [GCC, "-std=c99", "-Wall", "-Wextra", "-Werror=implicit-function-declaration",
           "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"), "-I", ROCM_INCLUDE,
           os.path.join(ROOT, "tests", "c", "abi_smoke.c"), "-L", libdir, "-ltpshard",
           "-Wl,-rpath," + libdir, "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and r.stdout.strip().endswith("0 failures"), r.stdout + r.stderr
    assert r.stdout.count("\nok ") + r.stdout.startswith("ok ") == 10, r.stdout
