"""Pins of the host C++ reference of the KV-outer reverse index and scheduler
(oracle/kv_schedule.cpp; "MSA 为什么采用 KV-outer Sparse Attention Forward",
sections 5 and 7).

* its brute-force checker (oracle/kv_schedule_check.cpp: the slot of every
  entry from a pairwise count, every count, row pointer, edge and chunk from
  the definitions) passes on 192 shapes, built with AddressSanitizer and
  UndefinedBehaviorSanitizer so an out-of-bounds access or overflow fails;
* the checker is not vacuous: each planted mistake in a copy of the reference
  (slots by position, the causal rule off by one, chunks one edge too long,
  a dropped edge) makes it fail;
* a small example worked out by hand;
* the slot counts and which slots hold a non-empty partial agree with the
  independent Python oracle (oracle.kvouter_partials).
"""

import os
import shutil
import subprocess

import numpy as np
import pytest

import oracle
from oracle import kv_schedule

pytestmark = pytest.mark.skipif(shutil.which("g++") is None, reason="needs the host g++")

SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]


def _compile_checker(tmp_path, source, flags):
    exe = str(tmp_path / "kv_check")
    subprocess.run(["g++", "-std=c++17", "-O1", "-g", *flags, source, kv_schedule.CHECKER, "-o", exe], check=True,
                   capture_output=True, text=True)
    return exe


def test_checker_passes_under_sanitizers(tmp_path):
    exe = _compile_checker(tmp_path, kv_schedule.SOURCE, SAN)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-4000:]
    assert r.stdout.strip() == "ok 192 cases"


MUTANTS = {
    "slots_by_position": ("std::sort(valid.begin(), valid.end());", ";"),
    "causal_off_by_one": ("(int64_t)blk * BK > i", "(int64_t)blk * BK >= i"),
    "chunk_one_too_long": ("std::min(n, c0 + cap)", "std::min(n, c0 + cap + 1)"),
    "edge_dropped": ("for (size_t s = 0; s < valid.size(); ++s) {", "for (size_t s = 0; s + 1 < valid.size(); ++s) {"),
}


@pytest.mark.parametrize("name", list(MUTANTS))
def test_checker_catches_planted_mistakes(tmp_path, name):
    old, new = MUTANTS[name]
    text = open(kv_schedule.SOURCE).read()
    assert text.count(old) == 1, "the mutation site moved"
    src = tmp_path / "kv_schedule_mutant.cpp"
    src.write_text(text.replace(old, new))
    exe = _compile_checker(tmp_path, str(src), [])
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300)
    assert r.returncode != 0 and "ok " not in r.stdout, name + " was not caught"


def test_hand_worked_example():
    """B = 1, N = 5, one KV head, k = 3, BK = 2 (blocks {0,1}, {2,3}, {4}),
    causal, cap = 2.  Rows of q2k and their slots (increasing block order,
    ties by position):
      i=0: [0]      -> slot 0 = block 0
      i=1: [1, 0]   -> block 0 slot 0, block 1 slot 1 (starts at 2 > 1: no edge)
      i=2: [1, 2, 0]-> block 0 slot 0, block 1 slot 1, block 2 slot 2 (4 > 2: no edge)
      i=3: [0, 1]   -> block 0 slot 0, block 1 slot 1
      i=4: [2, 2, 0]-> block 0 slot 0, block 2 twice: slots 1 and 2
    Reverse rows: block 0 gets (0,0) (1,0) (2,0) (3,0) (4,0); block 1 gets
    (2,1) (3,1); block 2 gets (4,1) (4,2).  With cap 2 block 0 splits into
    three chunks."""
    q2k = np.array([[0, -1, -1], [1, 0, -1], [1, 2, 0], [0, 1, -1], [2, 2, 0]], np.int32).reshape(1, 5, 1, 3)
    r = kv_schedule.reference(q2k, 2, causal=True, cap=2)
    assert r["nslot"].ravel().tolist() == [1, 2, 3, 2, 3]
    assert r["count"].tolist() == [5, 2, 2]
    assert r["rowptr"].tolist() == [0, 5, 7, 9]
    assert r["edges"].tolist() == [[0, 0], [1, 0], [2, 0], [3, 0], [4, 0], [2, 1], [3, 1], [4, 1], [4, 2]]
    assert r["chunks"].tolist() == [[0, 0, 2, 0], [0, 2, 4, 0], [0, 4, 5, 0], [1, 5, 7, 0], [2, 7, 9, 0]]
    assert not r["flagged"]
    # without the causal rule every valid entry is an edge
    r = kv_schedule.reference(q2k, 2, causal=False, cap=100)
    assert r["count"].tolist() == [5, 3, 3]
    assert r["chunks"].tolist() == [[0, 0, 5, 0], [1, 5, 8, 0], [2, 8, 11, 0]]
    # counts cut rows short; an id past the last block is skipped and flagged.
    # cnt = [1, 1, 2, 0, 3], row 4 = [2, 3, 0]: i=0 -> block 0; i=1 -> [1]
    # (no edge); i=2 -> [1, 2]: block 1 edge, block 2 none; i=3 -> nothing;
    # i=4 -> 3 skipped, block 0 slot 0 and block 2 slot 1 (4 <= 4).
    cnt = np.array([1, 1, 2, 0, 3], np.int32).reshape(1, 5, 1)
    bad = q2k.copy()
    bad[0, 4, 0, 1] = 3
    r = kv_schedule.reference(bad, 2, causal=True, q2k_cnt=cnt, cap=2)
    assert r["nslot"].ravel().tolist() == [1, 1, 2, 0, 2]
    assert r["count"].tolist() == [2, 1, 1] and r["flagged"]
    assert r["edges"].tolist() == [[0, 0], [4, 0], [2, 0], [4, 1]]


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("seed", [0, 1])
def test_agrees_with_python_oracle(seed, causal):
    """Independent code, same readings: nslot equals the Python oracle's, and a
    slot has an edge exactly when the oracle's partial over it is non-empty
    (finite log-sum-exp)."""
    rng = np.random.default_rng(seed)
    B, N, Hkv, G, ks, BK, D = 2, 37, 2, 2, 5, 4, 4
    NB = -(-N // BK)
    q2k = rng.integers(-1, NB, size=(B, N, Hkv, ks)).astype(np.int32)
    cnt = rng.integers(0, ks + 1, size=(B, N, Hkv)).astype(np.int32)
    q = rng.standard_normal((B, N, Hkv * G, D))
    k = rng.standard_normal((B, N, Hkv, D))
    v = rng.standard_normal((B, N, Hkv, D))
    _, lse, nslot = oracle.kvouter_partials(q, k, v, q2k, BK, causal=causal, q2k_cnt=cnt)
    r = kv_schedule.reference(q2k, BK, causal=causal, q2k_cnt=cnt, cap=3)
    assert np.array_equal(r["nslot"], nslot)
    has_edge = np.zeros((B, ks, N, Hkv), bool)
    rowid = np.repeat(np.arange(len(r["count"])), r["count"])
    b_of_row = rowid // (Hkv * NB)
    r_of_row = (rowid // NB) % Hkv
    has_edge[b_of_row, r["edges"][:, 1], r["edges"][:, 0], r_of_row] = True
    finite = np.isfinite(lse[..., ::G])       # one head per KV group: [B, ks, N, Hkv]
    assert np.array_equal(has_edge, finite)
