"""CPU check of the decode kernel's code-unpack plans (host logic, no GPU).

The decode kernel feeds b-bit codes to the MFMA as fp16 subnormals cut out of the packed
words with a shift and a mask per pair of codes. This compiles the kernel's own key and
value plans (code_plans.h) for the host and checks, for every width 2..8, that slot k of
step s holds code[chan(s, k)] << exp(s, k), inside the 10-bit mantissa, that every element
of a group is used exactly once, that the value plans' exponents repeat every two steps
(one weight operand serves every chunk), and that 2- to 4-bit codes sit at mantissa bit 2 or
above (4 or above for 2 bits), where the MFMA sums them with little error. It also checks
that the value plans read every stream in the order the cache format (tests/cache_format.py)
stores it.
"""
import os
import subprocess

import pytest

from tests import cache_format as F

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "mixed_precision_quantized_kvq_amd", "csrc")
HIPCC = "/opt/rocm/bin/hipcc"


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not installed")
def test_unpack_plans(tmp_path):
    exe = tmp_path / "unpack_plans_check"
    cmd = [HIPCC, "-std=c++20", "--offload-arch=gfx950", "-O1", "-I", os.path.join(ROOT, "include"),
           "-I", CSRC, "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           os.path.join(ROOT, "tests", "unpack_plans_check.hip"), "-o", str(exe)]
    subprocess.run(cmd, check=True, capture_output=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.count(": 0 mismatches") == 14, r.stdout
    # the value plans read each stream in the order the cache format stores it
    seen = set()
    for line in r.stdout.splitlines():
        if line.startswith("value stream order B="):
            head, vals = line.split(":")
            b = int(head.split("=")[1])
            assert [int(x) for x in vals.split()] == F.VALUE_STREAM_POS[b], b
            seen.add(b)
    assert seen == set(range(2, 9)), seen
