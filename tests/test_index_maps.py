"""The kernels' integer index maps, checked on the CPU.

aware_tiling_amd/csrc/index_maps.h holds the LDS swizzles, the key order of
transposed value reads, the workgroup remap and the per-lane offsets of
the tile copies and operand reads; the kernels call these functions.
tests/index/index_check.cpp enumerates every lane, row, tile and stage at
the compiled tile shapes and checks bounds, bijections, the bank-conflict
properties the comments state, and (simulating the transposed LDS read)
that each lane's operand holds the elements the MFMA layout needs.  Each
mutant below breaks one map in a copy of the header; the checker must
reject every one.
"""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "aware_tiling_amd", "csrc")
SRC = os.path.join(ROOT, "tests", "index", "index_check.cpp")


def _build_and_run(include_dir, tmp_path, name):
    exe = str(tmp_path / name)
    subprocess.run(["g++", "-std=c++17", "-O1", "-Wall", "-Werror", f"-I{include_dir}", SRC, "-o",
                    exe], check=True, capture_output=True, text=True)
    return subprocess.run([exe], capture_output=True, text=True, timeout=300)


def test_index_maps_hold(tmp_path):
    r = _build_and_run(CSRC, tmp_path, "index_check")
    assert r.returncode == 0, r.stderr
    assert "checks passed" in r.stdout


MUTANTS = [
    ("chunk_swizzle_drops_bit3", "    return row & 15;", "    return row & 7;"),
    ("vtr_swizzle_one_bit", "    return 4 * (row & 3);", "    return 4 * (row & 1);"),
    ("dual_swizzle_low_bits", "    return ((row & 3) << 2) | ((row >> 2) & 3);",
     "    return ((row & 3) << 2) | ((row >> 2) & 1);"),
    ("xcd_remap_wrong_shift", "return (w & 7) * per + (w >> 3);", "return (w & 7) * per + (w >> 2);"),
    ("copy_src_next_row_swizzle", "return (uint32_t)(row * D + (phys ^ SWZ(row)) * 8) * 2u;",
     "return (uint32_t)(row * D + (phys ^ SWZ(row + 1)) * 8) * 2u;"),
    ("tr_row_wrong_half", "return 8 * piece + 4 * ((lane >> 4) >> 1) + ((lane & 15) >> 2);",
     "return 8 * piece + 4 * ((lane >> 4) & 1) + ((lane & 15) >> 2);"),
    ("tr_col_wrong_lanes", "16 * ((lane >> 4) & 1) + 4 * (lane & 3);",
     "16 * ((lane >> 4) & 1) + 4 * ((lane >> 2) & 3);"),
    ("vt_key_pos_wrong_bit", "((k & 8) >> 1);", "((k & 8) >> 2);"),
    ("tile_elem_drops_bit2", "+ (col & 7);", "+ (col & 3);"),
    ("row_chunk_unswizzled", "return row * D + ((chunk ^ SWZ(row)) * 8);", "return row * D + chunk * 8;"),
]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_index_mutant_caught(name, old, new, tmp_path):
    inc = tmp_path / "inc"
    inc.mkdir()
    text = open(os.path.join(CSRC, "index_maps.h")).read()
    assert text.count(old) == 1, f"mutation site not found once: {old}"
    (inc / "index_maps.h").write_text(text.replace(old, new))
    r = _build_and_run(str(inc), tmp_path, "index_check_" + name)
    assert r.returncode == 1 and "FAILED" in r.stderr, f"mutant {name} not caught: {r.stdout}"
