"""Pins for the oracle's pooling, routing matrix and TopK (CPU only)."""

import itertools
import math

import numpy as np
import pytest

import oracle


def _hand_example(golden):
    """The D=2 example: block A's queries and block B's keys, per time slice."""
    g = golden("vsa_hand_example_d2.txt")
    Q = np.zeros((1, 64, 1, 2))
    K = np.zeros((1, 64, 1, 2))
    for t in range(4):
        qa0, qa1, kb0, kb1 = map(float, g["slice_%d" % t])
        for y in range(2):
            for x in range(2):
                Q[0, t * 16 + y * 4 + x, 0] = (qa0, qa1)          # block A: x in 0..1
                K[0, t * 16 + y * 4 + (x + 2), 0] = (kb0, kb1)    # block B: x in 2..3
    return g, Q, K


def test_hand_example_pool_and_route(golden):
    g, Q, K = _hand_example(golden)
    tab = oracle.tile_index(4, 4, 4, 4, 2, 2)
    qbar = oracle.pool_blocks(Q, tab["perm"], tab["block_len"], tab["M"])
    kbar = oracle.pool_blocks(K, tab["perm"], tab["block_len"], tab["M"])
    assert qbar[0, 0, 0].tolist() == [float(x) for x in g["qbar_A"]]
    assert kbar[0, 0, 1].tolist() == [float(x) for x in g["kbar_B"]]
    E = oracle.routing_matrix(qbar, kbar)
    assert abs(E[0, 0, 0, 1] - float(g["E_AB"][0])) < 1e-15
    assert abs(E[0, 0, 0, 1] - 3.0 / math.sqrt(2.0)) < 1e-15


@pytest.mark.parametrize("geom", [(5, 3, 4, 4, 2, 2), (6, 5, 7, 4, 4, 4)])
def test_mean_dot_identity_brute_force(geom):
    """E_ij = (1/(n_i n_j sqrt(D))) sum_a sum_b q_a.k_b over block members."""
    T, H, W, bT, bH, bW = geom
    rng = np.random.default_rng(7)
    N, h, D = T * H * W, 2, 5
    Q = rng.standard_normal((1, N, h, D))
    K = rng.standard_normal((1, N, h, D))
    tab = oracle.tile_index(*geom)
    M, J = tab["M"], tab["J"]
    E = oracle.routing_matrix(oracle.pool_blocks(Q, tab["perm"], tab["block_len"], M),
                              oracle.pool_blocks(K, tab["perm"], tab["block_len"], M))
    # membership from coordinates, independent of the packing tables
    JH, JW = -(-H // bH), -(-W // bW)
    block_of = np.empty(N, dtype=np.int64)
    for tok in range(N):
        t, rem = divmod(tok, H * W)
        y, x = divmod(rem, W)
        block_of[tok] = ((t // bT) * JH + y // bH) * JW + x // bW
    for hh in range(h):
        for i, j in itertools.product(range(J), repeat=2):
            qa = np.nonzero(block_of == i)[0]
            kb = np.nonzero(block_of == j)[0]
            tot = 0.0
            for a in qa:
                for b in kb:
                    tot += float(np.dot(Q[0, a, hh], K[0, b, hh]))
            ref = tot / (len(qa) * len(kb) * math.sqrt(D))
            assert abs(E[0, hh, i, j] - ref) < 1e-12


def test_pool_divides_by_true_length():
    tab = oracle.tile_index(5, 3, 4, 4, 2, 2)
    X = np.ones((1, 60, 3, 4))
    xbar = oracle.pool_blocks(X, tab["perm"], tab["block_len"], tab["M"])
    assert np.array_equal(xbar, np.ones_like(xbar))


def test_topk_page_example(golden):
    g = golden("vsa_topk_example.txt")
    E = np.array([[float(x) for x in g["scores_A"]]])
    idx, num, gap = oracle.select_topk(E, int(g["keep"][0]), kmax=4)
    assert idx[0].tolist() == [int(x) for x in g["q2k_idx_A"]]
    assert num[0] == int(g["q2k_num_A"][0])
    assert abs(gap[0] - (2.4 - 0.2)) < 1e-12


def _textbook_topk(row, R):
    order = sorted(range(len(row)), key=lambda j: (-row[j], j))
    return sorted(order[:R])


@pytest.mark.parametrize("J,R", [(4, 2), (9, 1), (9, 9), (33, 5), (64, 17)])
def test_topk_against_sorted_with_ties(J, R):
    rng = np.random.default_rng(J * 100 + R)
    E = rng.integers(-3, 4, size=(3, 5, J)).astype(np.float64)   # many exact ties
    idx, num, gap = oracle.select_topk(E, R, kmax=J)
    for a in range(3):
        for b in range(5):
            row = E[a, b].tolist()
            assert idx[a, b, :R].tolist() == _textbook_topk(row, R)
            assert (idx[a, b, R:] == -1).all()
            assert num[a, b] == R
            desc = sorted(row, reverse=True)
            assert gap[a, b] == (desc[R - 1] - desc[R] if R < J else np.inf)


def test_topk_special_cases():
    rng = np.random.default_rng(3)
    E = rng.standard_normal((4, 11))
    idx, _, _ = oracle.select_topk(E, 11)
    assert (idx == np.arange(11)).all()
    idx, _, _ = oracle.select_topk(E, 1)
    assert (idx[:, 0] == np.argmax(E, axis=-1)).all()
    with pytest.raises(ValueError):
        oracle.select_topk(E, 12)
    with pytest.raises(ValueError):
        oracle.select_topk(E, 3, kmax=2)
