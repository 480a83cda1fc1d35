"""Pins for the oracle's coarse pooled-V branch (CPU only).

Independent references: torch's scaled_dot_product_attention in float64 (the
one-token-block case is dense attention), closed forms (equal scores give the
mean, a dominant score selects one block, a hand-computed two-block row) and a
per-token brute force of the gated broadcast.
"""

import math

import numpy as np
import torch

import oracle


def test_one_token_blocks_give_dense_attention():
    """Blocks of one token: V_bar = V and E = Q K^T / sqrt(D), so the coarse
    branch is dense attention over all tokens."""
    rng = np.random.default_rng(21)
    T, H, W, h, D = 3, 4, 5, 2, 8
    N = T * H * W
    Q, K, V = (rng.standard_normal((1, N, h, D)) for _ in range(3))
    tab = oracle.tile_index(T, H, W, 1, 1, 1)
    pb = lambda X: oracle.pool_blocks(X, tab["perm"], tab["block_len"], tab["M"])
    C = oracle.coarse_attention(oracle.routing_matrix(pb(Q), pb(K)), pb(V))
    for hh in range(h):
        dense = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(Q[0, :, hh])[None, None], torch.from_numpy(K[0, :, hh])[None, None],
            torch.from_numpy(V[0, :, hh])[None, None])[0, 0].numpy()
        # block i holds token perm[i]
        assert np.max(np.abs(C[0, hh] - dense[tab["perm"]])) < 1e-12


def test_equal_scores_give_the_block_mean():
    rng = np.random.default_rng(22)
    vbar = rng.standard_normal((1, 2, 7, 5))
    E = np.full((1, 2, 7, 7), 0.37)
    C = oracle.coarse_attention(E, vbar)
    assert np.max(np.abs(C - vbar.mean(axis=2, keepdims=True))) < 1e-14


def test_dominant_score_selects_its_block():
    rng = np.random.default_rng(23)
    vbar = rng.standard_normal((1, 1, 6, 4))
    E = rng.standard_normal((1, 1, 6, 6))
    top = [3, 0, 5, 1, 1, 2]
    for i, j in enumerate(top):
        E[0, 0, i, j] += 1e3
    C = oracle.coarse_attention(E, vbar)
    assert np.max(np.abs(C[0, 0] - vbar[0, 0, top])) < 1e-12


def test_hand_row():
    """Scores [0, ln 3] weigh the two blocks 1/4 and 3/4."""
    vbar = np.array([2.0, -6.0]).reshape(1, 1, 2, 1)
    E = np.array([[0.0, math.log(3.0)], [math.log(3.0), 0.0]]).reshape(1, 1, 2, 2)
    C = oracle.coarse_attention(E, vbar)
    assert abs(C[0, 0, 0, 0] - (0.25 * 2.0 + 0.75 * -6.0)) < 1e-15
    assert abs(C[0, 0, 1, 0] - (0.75 * 2.0 + 0.25 * -6.0)) < 1e-15


def test_gated_broadcast_brute_force():
    rng = np.random.default_rng(24)
    T, H, W, h, D = 5, 3, 4, 2, 6
    N = T * H * W
    tab = oracle.tile_index(T, H, W, 4, 2, 2)
    O = rng.standard_normal((1, N, h, D))
    C = rng.standard_normal((1, h, tab["J"], D))
    g = rng.standard_normal((h, D))
    got = oracle.add_coarse(O, C, g, tab["perm"], tab["block_len"], tab["M"])
    # brute force from token coordinates, independent of the packing tables
    JH, JW = -(-H // 2), -(-W // 2)
    for tok in range(N):
        t, rem = divmod(tok, H * W)
        y, x = divmod(rem, W)
        i = ((t // 4) * JH + y // 2) * JW + x // 2
        assert np.allclose(got[0, tok], O[0, tok] + g * C[0, :, i], atol=1e-15, rtol=0)
    assert np.array_equal(oracle.add_coarse(O, C, np.zeros((h, D)), tab["perm"], tab["block_len"], tab["M"]), O)
