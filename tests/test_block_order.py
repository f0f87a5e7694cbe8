"""CPU check of the forward kernels' block order (block_order.h).

tests/block_order_check.cpp maps every block id of seven shapes and checks
that the map is a bijection onto (batch, K/V head, head, query block), that
it equals a plain-division reference, and, on the longest-first path, that a
group stays on one XCD and each band runs heaviest first; and that the
run-time tail of tail_queue.h runs every block once.  Planted mistakes
in a copy of the header must make it fail.
"""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "transformer_self_attention_attn_amd", "csrc")
CHECK = os.path.join(ROOT, "tests", "block_order_check.cpp")
HEADER = open(os.path.join(CSRC, "block_order.h")).read()

pytestmark = pytest.mark.skipif(shutil.which("g++") is None,
                                reason="needs a host C++ compiler")


def build_and_run(tmp_path, header_text=None):
    inc = str(tmp_path / "inc")
    os.makedirs(inc, exist_ok=True)
    shutil.copy(os.path.join(CSRC, "fastdiv.h"), inc)
    shutil.copy(os.path.join(CSRC, "tail_queue.h"), inc)
    with open(os.path.join(inc, "block_order.h"), "w") as f:
        f.write(HEADER if header_text is None else header_text)
    exe = str(tmp_path / "block_order_check")
    subprocess.run(["g++", "-std=c++17", "-O2", "-I", inc, "-o", exe, CHECK],
                   check=True, capture_output=True, text=True)
    return subprocess.run([exe], capture_output=True, text=True)


def test_block_order(tmp_path):
    r = build_and_run(tmp_path)
    assert r.returncode == 0, r.stdout
    assert "all checks passed" in r.stdout


MUTANTS = {
    # the head within the group taken from the wrong remainder
    "head_index": ("    hh = r2 - r2g * o.G;", "    hh = r2g;"),
    # causal blocks lightest first
    "causal_order": ("pos.qb = o.causal ? (o.nqb - 1 - qrank) : qrank;",
                     "pos.qb = qrank;"),
    # an XCD's groups overlapping the next XCD's
    "group_base": ("    grp = xcd * o.gpx + gi;", "    grp = xcd + gi;"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_order_mistake_is_caught(tmp_path, name):
    old, new = MUTANTS[name]
    assert old in HEADER, name
    r = build_and_run(tmp_path, HEADER.replace(old, new, 1))
    assert r.returncode != 0, f"{name} not caught:\n{r.stdout}"
    assert "FAIL" in r.stdout
