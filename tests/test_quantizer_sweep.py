"""The store kernels' code computation (quantizer.h, compiled for the host)
against the codec's definition, on the CPU, for every fp16 scale.

The kernels avoid a division per element: a fused multiply-add by the
reciprocal of the scale is exact except on exact ties, which are flagged and
redone by an exact routine.  tests/quantizer_sweep.hip runs that code on the
host over every scale an absmax can give (INT8 symmetric: every reachable
element; INT4 and INT8 asymmetric: every scale with a main set of zero
points and every zero point on a stride of scales) and compares each code
with clamp(rint(fp32(fp32(x / s) + zp))), the oracle's reading of yunthe.com
"quantization principle" Q(x).  A wrong tie rule, a missed flag or a dropped
clamp fails it.
"""

import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = "/opt/rocm/bin/hipcc"


@pytest.fixture(scope="module")
def sweep_bin(tmp_path_factory):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    out = str(tmp_path_factory.mktemp("qsweep") / "quantizer_sweep")
    cmd = [HIPCC, "-x", "hip", "--offload-host-only", "-O2", "-ffp-contract=off", "-fno-fast-math",
           "-std=c++17", "-I", os.path.join(ROOT, "paged_block_quantized_amd", "csrc"),
           "-I", os.path.join(ROOT, "include"), os.path.join(ROOT, "tests", "quantizer_sweep.hip"),
           "-o", out, "-lpthread"]
    subprocess.run(cmd, check=True, capture_output=True)
    return out


@pytest.mark.parametrize("mode", ["i8", "i4", "i8a"])
def test_quantizer_matches_definition_all_scales(sweep_bin, mode):
    threads = str(max(1, min(16, os.cpu_count() or 1)))
    r = subprocess.run([sweep_bin, mode, threads], capture_output=True, text=True, timeout=600)
    print(r.stdout, r.stderr)
    assert r.returncode == 0, r.stdout + r.stderr
    fields = dict(kv.split("=") for kv in r.stdout.split()[1:])
    assert int(fields["bad_fast"]) == 0 and int(fields["bad_exact"]) == 0
    # the sweep reached the cases it is about: ties (flagged and redone) and
    # every scale
    assert int(fields["flagged"]) > 1000
    if mode == "i8":
        assert int(fields["scales"]) > 24000   # distinct fp16(a / 127), zero included
