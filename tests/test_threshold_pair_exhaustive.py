"""Exhaustive host check of the quantize kernel's fp32 threshold decisions
for 16-bit inputs (no GPU): the pair form (fp16) and the one-value T form
(bf16), every x in [-s, s] against every 16-bit significand of s, for the
NF2..NF5, FP4, Lloyd-Max and random 16- and 32-entry codebooks' switching
points.  A planted one-ulp shift of the pair threshold, and the other choice
of T, must both be caught.
"""

import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = [os.path.join(ROOT, "tests", "host", "pair_decision_check.cpp"),
       os.path.join(ROOT, "blockwise_bit_codebook_amd", "csrc", "codebook.cpp")]


def _build(tmp_path, name, defines=()):
    exe = str(tmp_path / name)
    cmd = ["g++", "-O2", "-std=c++17", "-ffp-contract=off", "-fno-fast-math", "-pthread",
           "-I", os.path.join(ROOT, "include")] + [f"-D{d}" for d in defines] + ["-o", exe] + SRC
    subprocess.run(cmd, check=True)
    return exe


def test_pair_decision_matches_division_rule(tmp_path):
    exe = _build(tmp_path, "pdc")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "mismatches 0" in r.stdout


def test_checker_catches_a_shifted_threshold(tmp_path):
    exe = _build(tmp_path, "pdc_planted", ["PLANT_ONE_ULP_SHIFT"])
    r = subprocess.run([exe, "quick"], capture_output=True, text=True, timeout=600)
    assert r.returncode != 0 and "mismatch x=" in r.stdout


def test_checker_catches_the_other_T(tmp_path):
    # the NF codebooks have switching points with a bf16 quotient inside
    # [p, u], where the choice of T matters
    exe = _build(tmp_path, "pdc_t_flip", ["PLANT_T_FLIP"])
    r = subprocess.run([exe], capture_output=True, text=True, timeout=600)
    assert r.returncode != 0 and "T mismatch x=" in r.stdout
