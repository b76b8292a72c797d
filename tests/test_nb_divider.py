"""Host check (no GPU) of the nested-state encoder's division of the exact
sum by the block count: a multiply-high by a host-computed constant must
equal integer division for every dividend below 2^63 and nb up to 2^36
(tests/host/nb_divider_check.cpp), and the checker must catch a multiplier
rounded the wrong way.
"""

import os
import subprocess

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "host", "nb_divider_check.cpp")
INC = os.path.join(ROOT, "blockwise_bit_codebook_amd", "csrc")


def _build(tmp_path, name, defines=()):
    exe = str(tmp_path / name)
    subprocess.run(["g++", "-O2", "-std=c++17", "-I", INC] + [f"-D{d}" for d in defines] + ["-o", exe, SRC],
                   check=True)
    return exe


def test_multiply_high_equals_division(tmp_path):
    r = subprocess.run([_build(tmp_path, "nbd")], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "mismatches 0" in r.stdout


def test_checker_catches_a_rounded_down_multiplier(tmp_path):
    r = subprocess.run([_build(tmp_path, "nbd_planted", ["PLANT_FLOOR_MAGIC"])], capture_output=True, text=True,
                       timeout=300)
    assert r.returncode != 0 and "mismatch nb=" in r.stdout
