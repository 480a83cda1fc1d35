"""Pins for the oracle's 3D tiling and keep budget (CPU only)."""

import math

import numpy as np
import pytest

import oracle


def test_teaching_grid_dims(golden):
    g = golden("vsa_teaching_grid.txt")
    T, H, W = map(int, g["grid"])
    bT, bH, bW = map(int, g["block"])
    assert oracle.tile_dims(T, H, W, bT, bH, bW) == (int(g["J"][0]), int(g["M"][0]))


def test_teaching_grid_block_A(golden):
    g = golden("vsa_teaching_grid.txt")
    tab = oracle.tile_index(4, 4, 4, 4, 2, 2)
    assert tab["perm"][:16].tolist() == [int(x) for x in g["block_A_members"]]


def test_teaching_grid_packed_order(golden):
    g = golden("vsa_teaching_grid.txt")
    tab = oracle.tile_index(4, 4, 4, 4, 2, 2)
    assert "".join(str(int(x)) for x in tab["perm"]) == g["packed_digits"][0]
    assert tab["block_len"].tolist() == [16, 16, 16, 16]
    # packed position 2 holds token 4, so token 4 goes back from position 2
    assert tab["perm"][2] == int(g["packed_pos_2_token"][0])
    assert tab["inv"][4] == 2


def _brute_force_tables(T, H, W, bT, bH, bW):
    """Block of every token from its coordinates; members in token-id order."""
    JT, JH, JW = -(-T // bT), -(-H // bH), -(-W // bW)
    groups = {}
    for tok in range(T * H * W):
        t, rem = divmod(tok, H * W)
        y, x = divmod(rem, W)
        b = ((t // bT) * JH + (y // bH)) * JW + (x // bW)
        groups.setdefault(b, []).append(tok)
    return [groups.get(b, []) for b in range(JT * JH * JW)]


@pytest.mark.parametrize("geom", [
    (5, 3, 4, 4, 2, 2),
    (4, 4, 4, 4, 2, 2),
    (7, 5, 9, 4, 4, 4),
    (30, 48, 80, 4, 4, 4),
    (3, 7, 2, 2, 3, 5),
])
def test_tiling_matches_brute_force(geom):
    T, H, W, bT, bH, bW = geom
    tab = oracle.tile_index(*geom)
    M = tab["M"]
    groups = _brute_force_tables(*geom)
    assert len(groups) == tab["J"]
    for b, members in enumerate(groups):
        n = len(members)
        assert tab["block_len"][b] == n
        assert tab["perm"][b * M: b * M + n].tolist() == members
        assert (tab["perm"][b * M + n: (b + 1) * M] == -1).all()
    valid = tab["perm"][tab["perm"] >= 0]
    assert np.array_equal(np.sort(valid), np.arange(T * H * W))
    assert np.array_equal(tab["perm"][tab["inv"]], np.arange(T * H * W))
    assert tab["block_len"].sum() == T * H * W


def test_edge_grid_sizes():
    # (5,3,4) in (4,2,2): one partial temporal slab and one partial row band
    tab = oracle.tile_index(5, 3, 4, 4, 2, 2)
    assert sorted(tab["block_len"].tolist(), reverse=True) == [16, 16, 8, 8, 4, 4, 2, 2]
    assert tab["block_len"].sum() == 60


def test_video_grid_edge_slab():
    tab = oracle.tile_index(30, 48, 80, 4, 4, 4)
    bl = tab["block_len"]
    assert tab["J"] == 1920 and tab["M"] == 64
    assert (bl == 64).sum() == 1680 and (bl == 32).sum() == 240
    assert (bl[-240:] == 32).all()


def test_keep_budget(golden):
    g = golden("vsa_topk_example.txt")
    assert oracle.keep_budget(float(g["budget_drop"][0]), int(g["budget_blocks"][0])) == int(g["budget_keep"][0])
    assert oracle.keep_budget(0.7, 10) == 3       # (1-0.7)*10 is 3.0000000000000004
    assert oracle.keep_budget(0.0, 17) == 17
    assert oracle.keep_budget(1.0, 17) == 1
    assert oracle.keep_budget(0.9, 1920) == 192
    assert oracle.keep_budget(0.75, 32) == 8
    for J in (1, 3, 10, 255):
        for s in (0.05, 0.33, 0.5, 0.9):
            assert oracle.keep_budget(s, J) == max(1, min(math.ceil(round((1 - s) * J, 9)), J))
