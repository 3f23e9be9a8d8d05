"""The GPU quantizers divide the 32 values of a block by one scale through a
shared correctly rounded reciprocal and two fma corrections. This CPU test
compiles tests/shared_divisor_check.c and checks that the resulting codes
equal those from IEEE division on the formats' operand domains."""
import os
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.fixture(scope="module")
def checker(tmp_path_factory):
    exe = str(tmp_path_factory.mktemp("divchk") / "shared_divisor_check")
    src = os.path.join(HERE, "shared_divisor_check.c")
    subprocess.run(["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-o", exe, src, "-lm"],
                   check=True)
    return exe


@pytest.mark.parametrize("seed", [1, 2])
def test_shared_divisor_codes_match_ieee_division(checker, seed):
    r = subprocess.run([checker, "20000000", str(seed)], capture_output=True, text=True)
    assert r.returncode == 0, r.stdout
    assert r.stdout.startswith("ok")
