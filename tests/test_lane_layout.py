"""CPU check of every lane's tile-load addressing (prefill, backward, FP8).

The kernels take each lane's source offset and the byte range of each
buffer resource from csrc/lane_layout.h; tests/lane_layout_check.cpp calls
the same functions on the host and checks, for every wavefront, lane and
load number, that reads stay inside their tile and resource, that LDS
writes stay inside their slot or sink, that each tile is covered once, and
that rows past the valid length are never in range.  This is the check that
a memory fault from loads past the end of K once called for.  Planted
mistakes in a copy of the header must make it fail.
"""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "transformer_self_attention_attn_amd", "csrc")
CHECK = os.path.join(ROOT, "tests", "lane_layout_check.cpp")

pytestmark = pytest.mark.skipif(shutil.which("g++") is None,
                                reason="needs a host C++ compiler")


def build_and_run(tmp_path, header_text=None):
    inc = CSRC
    if header_text is not None:
        inc = str(tmp_path / "inc")
        os.makedirs(inc, exist_ok=True)
        with open(os.path.join(inc, "lane_layout.h"), "w") as f:
            f.write(header_text)
    exe = str(tmp_path / "lane_check")
    subprocess.run(["g++", "-std=c++17", "-O1", "-I", inc, "-o", exe, CHECK],
                   check=True, capture_output=True, text=True)
    return subprocess.run([exe], capture_output=True, text=True)


def test_every_lane_stays_in_bounds(tmp_path):
    r = build_and_run(tmp_path)
    assert r.returncode == 0, r.stdout
    assert "all checks passed" in r.stdout


HEADER = open(os.path.join(CSRC, "lane_layout.h")).read()

MUTANTS = {
    # a K row's pad chunk reads the chunk past the row's end (the next
    # row's first, or past the tile for the last row)
    "prefill_k_pad_past_row": ("mfma_row(r) * D + (c < D / 8 ? c * 8 : 0)",
                               "mfma_row(r) * D + (c <= D / 8 ? c * 8 : 0)"),
    # V pad chunks read their own positions, past the row
    "prefill_v_pad_past_row": ("(unsigned)(r * D + (c < D / 8 ? c * 8 : 0)",
                               "(unsigned)(r * D + (c < D / 8 + 4 ? c * 8 : 0)"),
    # a tile's resource not clamped to the valid length
    "prefill_rsrc_unclamped": ("const int rows = rem - over;",
                               "const int rows = rem;"),
    # a chunk permutation wider than the row (d=128 rows have 16 chunks)
    "bwd_swz_past_row": ("return D == 128 ? 4 * (r & 3) +",
                         "return D == 128 ? 8 * (r & 3) +"),
    # K code rows of the FP8 tile one chunk off
    "fp8_k_row": ("return (unsigned)(row * D + 16 * c);",
                  "return (unsigned)(row * D + 16 * c + 16);"),
    # V^T code rows one row off
    "fp8_v_row": ("return (unsigned)(row * 64 + 16 * c);",
                  "return (unsigned)(row * 64 + 64 + 16 * c);"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_addressing_mistake_is_caught(tmp_path, name):
    old, new = MUTANTS[name]
    assert old in HEADER, name
    r = build_and_run(tmp_path, HEADER.replace(old, new, 1))
    assert r.returncode != 0, f"{name} not caught:\n{r.stdout}"
    assert "FAIL" in r.stdout
