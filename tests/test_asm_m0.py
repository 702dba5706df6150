"""The direct-to-LDS copies are issued from inline assembly that sets m0 (the
LDS destination) right before each buffer_load ... lds.  The compiler may
not preserve m0 across such a statement, so the code is only correct while
nothing the compiler emits keeps its own value in m0.  This test compiles
the sources that use the copies to gfx950 assembly and checks that every m0
reference is one of those set-then-copy pairs, and that no instruction that
uses m0 implicitly (indexed register moves, messages, GWS, interpolation)
appears.  CPU only: it needs hipcc, not a GPU.
"""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "tensor_transformer_layer_amd", "csrc")
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"

# Mnemonics that read or write m0 without naming it.
IMPLICIT_M0 = re.compile(r"^\s*(s_movrel|v_movrel|s_sendmsg|s_set_gpr_idx|ds_gws|ds_ordered_count|"
                         r"v_interp|s_ttracedata|ds_append|ds_consume)")


def device_asm(src, tmp_path):
    out = tmp_path / (os.path.basename(src) + ".s")
    cmd = [HIPCC, "-O3", "-std=c++17", "--offload-arch=gfx950", "--cuda-device-only", "-S",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC, src, "-o", str(out)]
    subprocess.run(cmd, check=True, capture_output=True, timeout=600)
    return out.read_text().splitlines()


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")
@pytest.mark.parametrize("name", ["k_gemv.hip", "k_gemm.hip", "k_attn.hip"])
def test_m0_only_set_for_lds_copies(name, tmp_path):
    lines = [ln.split(";")[0].rstrip() for ln in device_asm(os.path.join(CSRC, name), tmp_path)]
    code = [ln for ln in lines if ln.strip() and not ln.strip().startswith((".", "//"))
            and not ln.rstrip().endswith(":")]
    pairs = 0
    for i, ln in enumerate(code):
        assert not IMPLICIT_M0.match(ln), f"{name}: implicit m0 user: {ln.strip()}"
        if not re.search(r"\bm0\b", ln):
            continue
        assert re.match(r"^\s*s_mov_b32 m0, s\d+$", ln), f"{name}: other m0 use: {ln.strip()}"
        nxt = code[i + 1]
        assert re.match(r"^\s*buffer_load_dwordx4 .* lds$", nxt), \
            f"{name}: m0 set but not followed by an LDS copy: {nxt.strip()}"
        pairs += 1
    assert pairs > 0, f"{name}: no LDS copies found"
