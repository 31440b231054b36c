"""The block-list check of the list-checking build, on the host.

The function that libbsattn_checked.so runs on the device before block-sparse
attention (csrc/listcheck.h) is compiled here into a small host driver with
address and undefined-behaviour sanitizers; rows and bitmaps live in heap
arrays of exactly their size, so any read past them fails the run. Its
answers are compared with a set-based statement of the contract written
below: a list is `cnt` entries at the start of a row of `stride` slots, each
a KV block index in [0, nk), none repeated (vllm-omni PR #8335, Purpose:
the selector lists KV blocks, and their number, per query head and block).
"""
import os
import random
import subprocess

import pytest

from conftest import ROOT

CSRC = os.path.join(ROOT, "block_sparse_attention_blocks_amd", "csrc")
DRIVER = os.path.join(ROOT, "tests", "listcheck_driver.cpp")
OK, COUNT, RANGE, DUP = 0, 1, 2, 3


def expected(nk, stride, cnt, row):
    """(fault, slot) of the first violation in list order."""
    if cnt < 0 or cnt > stride:
        return COUNT, -1
    seen = set()
    for j, e in enumerate(row[:cnt]):
        if not 0 <= e < nk:
            return RANGE, j
        if e in seen:
            return DUP, j
        seen.add(e)
    return OK, -1


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    exe = str(tmp_path_factory.mktemp("listcheck") / "listcheck_driver")
    subprocess.run(["g++", "-std=c++17", "-O1", "-g", "-Wall", "-Werror",
                    "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
                    "-fno-omit-frame-pointer", "-I", CSRC, DRIVER, "-o", exe], check=True)
    return exe


def run(driver, cases):
    text = "".join(f"{nk} {stride} {cnt} {' '.join(map(str, row))}\n" for nk, stride, cnt, row in cases)
    r = subprocess.run([driver], input=text, capture_output=True, text=True,
                       env=dict(os.environ, ASAN_OPTIONS="detect_leaks=1:halt_on_error=1",
                                UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1"))
    assert r.returncode == 0, r.stderr[-3000:]
    assert "Sanitizer" not in r.stderr and "runtime error" not in r.stderr, r.stderr[-3000:]
    out = [tuple(map(int, line.split())) for line in r.stdout.splitlines()]
    assert len(out) == len(cases)
    return out


HAND = [
    # nk, stride, cnt, row                        fault, slot
    ((764, 4, 4, [0, 5, 9, 763]), (OK, -1)),       # ascending, last block included
    ((764, 4, 4, [763, 0, 9, 5]), (OK, -1)),       # order does not matter
    ((764, 4, 3, [0, 5, 9, 9]), (OK, -1)),         # slot past cnt is not read
    ((764, 4, 0, [-1, -1, -1, -1]), (OK, -1)),     # empty list
    ((764, 4, 4, [0, 5, 764, 1]), (RANGE, 2)),     # entry == nk
    ((764, 4, 4, [-1, 5, 6, 1]), (RANGE, 0)),      # negative entry
    ((764, 4, 4, [3, 5, 3, 1]), (DUP, 2)),         # repeat, not adjacent
    ((764, 4, 4, [3, 3, 900, 1]), (DUP, 1)),       # first violation wins
    ((764, 4, 5, [0, 1, 2, 3]), (COUNT, -1)),      # cnt > stride
    ((764, 4, -1, [0, 1, 2, 3]), (COUNT, -1)),     # cnt < 0
    ((33, 3, 3, [32, 31, 0]), (OK, -1)),           # bitmap word boundary
    ((33, 3, 3, [32, 31, 32]), (DUP, 2)),
    ((4096, 3, 3, [4095, 4064, 4095]), (DUP, 2)),  # last bitmap bit
    ((5000, 3, 3, [4999, 4096, 4999]), (DUP, 2)),  # past the device bitmap size
    ((1, 1, 1, [0]), (OK, -1)),
    ((1, 2, 2, [0, 0]), (DUP, 1)),
]


def test_hand_cases(driver):
    out = run(driver, [c for c, _ in HAND])
    for (case, want), got in zip(HAND, out):
        assert got[:2] == want, (case, got)
        assert got[2:] == want, (case, got)   # pairwise path agrees
        assert expected(*case) == want         # the statement above agrees


def test_random_rows(driver):
    rng = random.Random(20261202)
    cases = []
    for _ in range(3000):
        nk = rng.choice([1, 2, 31, 32, 33, 64, 191, 764, 1354, 4096, 4097, 6000])
        stride = rng.randint(1, min(nk + 3, 400))
        cnt = rng.choice([rng.randint(0, stride), stride, stride + 1, -1, 0])
        pool = list(range(nk))
        rng.shuffle(pool)
        row = pool[:stride] + [0] * max(0, stride - nk)
        kind = rng.random()
        if kind < 0.25 and cnt > 1 and cnt <= stride:   # plant a repeat
            a, b = sorted(rng.sample(range(cnt), 2))
            row[b] = row[a]
        elif kind < 0.5 and cnt > 0 and cnt <= stride:  # plant an out-of-range entry
            row[rng.randrange(cnt)] = rng.choice([-5, -1, nk, nk + 7, 2 ** 31 - 1, -2 ** 31])
        cases.append((nk, stride, cnt, row))
    out = run(driver, cases)
    faults = set()
    for case, got in zip(cases, out):
        want = expected(*case)
        assert got[:2] == want and got[2:] == want, (case[:3], got, want)
        faults.add(want[0])
    assert faults == {OK, COUNT, RANGE, DUP}
