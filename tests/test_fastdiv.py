"""CPU check of the prefill's division by launch-fixed divisors (fastdiv.h).

tests/fastdiv_check.cpp compares udiv(n, make_udiv(d)) with n / d over every
divisor up to 5000 (dividends around each multiple, up to 2^31 - 1) and
sampled divisors up to 2^31 - 1.  Planted mistakes in a copy of the header
must make it fail.
"""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "transformer_self_attention_attn_amd", "csrc")
CHECK = os.path.join(ROOT, "tests", "fastdiv_check.cpp")
HEADER = open(os.path.join(CSRC, "fastdiv.h")).read()

pytestmark = pytest.mark.skipif(shutil.which("g++") is None,
                                reason="needs a host C++ compiler")


def build_and_run(tmp_path, header_text=None):
    inc = CSRC
    if header_text is not None:
        inc = str(tmp_path / "inc")
        os.makedirs(inc, exist_ok=True)
        with open(os.path.join(inc, "fastdiv.h"), "w") as f:
            f.write(header_text)
    exe = str(tmp_path / "fastdiv_check")
    subprocess.run(["g++", "-std=c++17", "-O2", "-I", inc, "-o", exe, CHECK],
                   check=True, capture_output=True, text=True)
    return subprocess.run([exe], capture_output=True, text=True)


def test_division_matches_integer_division(tmp_path):
    r = build_and_run(tmp_path)
    assert r.returncode == 0, r.stdout
    assert "all checks passed" in r.stdout


MUTANTS = {
    # the multiplier rounded down instead of up
    "floor_multiplier": ("(num + (unsigned long long)d - 1) / (unsigned long long)d",
                         "num / (unsigned long long)d"),
    # one bit of shift too few
    "short_shift": ("return UDiv{(unsigned)m, 31 + l};",
                    "return UDiv{(unsigned)(m >> 1), 30 + l};"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_division_mistake_is_caught(tmp_path, name):
    old, new = MUTANTS[name]
    assert old in HEADER, name
    r = build_and_run(tmp_path, HEADER.replace(old, new, 1))
    assert r.returncode != 0, f"{name} not caught:\n{r.stdout}"
    assert "FAIL" in r.stdout
