"""Planted mistakes in the oracle must be caught by its pins.  CPU only.

Each mutant is the oracle source compiled with ORACLE_MUTANT=k (a dropped
scale, a wrong GQA head map, an extra or shifted slot, a flipped exponent sign,
K used as V, a dropped denominator term, unnormalized partials, overlapping
partitions, a merge without exp_sum weights, a dropped causal diagonal,
top-left causal alignment, a shifted query row, a transposed query index,
FP8 ties away from zero, a wrong FP8 scale, a late append position, FP8
subnormals dropped, a swapped x-packed K index, a token-granular length read
as the end offset).
Every build runs the pin suite in a child process (a mutant may crash); the
test requires at least one failing pin or a crash for each.
"""
import json
import os
import subprocess
import sys

import pytest

import oracle

MUTANTS = {
    1: "scale dropped",
    2: "GQA head map h % H_kv",
    3: "one slot past the sequence",
    4: "slot index shifted",
    5: "exponent sign flipped",
    6: "K used as V",
    7: "first denominator term dropped",
    8: "partials left unnormalized",
    9: "partitions overlap by one token",
    10: "merge ignores exp_sums",
    11: "causal diagonal dropped",
    12: "causal mask aligned top-left",
    13: "query row shifted",
    14: "query index transposed",
    15: "FP8 ties rounded away from zero",
    16: "FP8 scale from the wrong largest magnitude (240)",
    17: "append one position late",
    18: "FP8 subnormals read as zero",
    19: "x-packed K index with chunk and lane swapped",
    20: "token-granular length read as the end offset",
}

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.parametrize("mutant", sorted(MUTANTS))
def test_pins_reject_mutant(tmp_path, mutant):
    lib = str(tmp_path / f"liboracle_m{mutant}.so")
    oracle.compile_library(lib, mutant=mutant)
    proc = subprocess.run([sys.executable, os.path.join(ROOT, "tests", "oracle_pins.py"), lib],
                          capture_output=True, text=True, timeout=300, cwd=ROOT)
    if proc.returncode != 0:
        return  # the mutant crashed a pin: rejected
    failed = json.loads(proc.stdout.strip().splitlines()[-1])["failed"]
    assert failed, f"mutant {mutant} ({MUTANTS[mutant]}) passed every pin"
