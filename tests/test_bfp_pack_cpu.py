"""The prefill path's packed y format (pack_bfp4 in csrc/flint_internal.hpp),
compiled for the host and checked bit for bit against the format's plain
definition on 6 million blocks: normal values over many binades, arbitrary bit
patterns (NaN, infinities, subnormals), values at and next to the rounding
halfway points and the clamp at 2^13.  The device compiler fuses the scaling
and the rounding offset into one multiply-add; the second build does the same
on the host (the scaling is by a power of two, so the product is exact and the
fused form rounds identically).  CPU only.
"""
import os
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SRC = os.path.join(ROOT, "tests", "bfp_pack_check.cpp")


@pytest.mark.parametrize("fused", [False, True], ids=["separate", "fused-multiply-add"])
def test_pack_bfp4_matches_format_definition(fused):
    if not os.path.exists(HIPCC):
        pytest.skip("needs hipcc")
    extra = ["-mfma", "-ffp-contract=fast"] if fused else ["-ffp-contract=off"]
    with tempfile.TemporaryDirectory() as tmp:
        exe = os.path.join(tmp, "bfp_check")
        subprocess.run([HIPCC, "-x", "hip", "--cuda-host-only", "-O2", "-std=c++17", *extra,
                        "-I", os.path.join(ROOT, "include"),
                        "-I", os.path.join(ROOT, "sparse_moe_transformer_gemv_amd", "csrc"), SRC, "-o", exe],
                       check=True, capture_output=True)
        p = subprocess.run([exe], capture_output=True, text=True, timeout=300)
    assert p.returncode == 0, p.stdout + p.stderr
    assert "mismatches 0" in p.stdout, p.stdout
