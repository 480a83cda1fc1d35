"""Pins for the oracle's Spark-Reblock reordering (CPU only).

Independent references: explicit score profiles for the cross-moment cosine
identity, a hand-computed second moment, numpy's Cholesky product, torch's
float64 SDPA for permutation invariance, numpy's eigh for the principal axis,
the capacity rule counted by hand, and an interleaved two-cluster case the
equal-capacity split must separate.
"""

import numpy as np
import torch

import oracle
from oracle import reblock as rb


def test_second_moment_hand_example():
    Q = np.array([[1.0, 2.0], [3.0, 4.0]]).reshape(1, 2, 1, 2)
    assert np.array_equal(rb.second_moment(Q)[0, 0], np.array([[5.0, 7.0], [7.0, 10.0]]))


def test_factor_reproduces_the_ridged_moment():
    rng = np.random.default_rng(50)
    M = rb.second_moment(rng.standard_normal((2, 40, 3, 6)))
    L = rb.metric_factor(M, ridge=1e-3)
    assert np.allclose(np.triu(L, 1), 0.0)
    tr = np.trace(M, axis1=-2, axis2=-1)[..., None, None]
    assert np.max(np.abs(L @ np.swapaxes(L, -1, -2) - (M + 1e-3 * tr / 6 * np.eye(6)))) < 1e-12


def test_zero_trace_and_zero_key():
    Q = np.zeros((1, 5, 1, 3))
    L = rb.metric_factor(rb.second_moment(Q), ridge=0.25)
    assert np.allclose(L[0, 0], 0.5 * np.eye(3))
    K = np.ones((1, 5, 1, 3))
    K[0, 2] = 0.0
    U = rb.key_features(K, Q + 1.0)
    assert np.array_equal(U[0, 0, 2], np.zeros(3)) and np.all(np.isfinite(U))


def test_cosine_identity_with_score_profiles():
    """The cosine of two keys' features equals the cosine of their score
    profiles over all queries (no ridge: the identity is exact)."""
    rng = np.random.default_rng(51)
    B, N, h, D = 1, 300, 2, 8
    Q = rng.standard_normal((B, N, h, D))
    K = rng.standard_normal((B, N, h, D))
    U = rb.key_features(K, Q, ridge=0.0)
    for hh in range(h):
        S = Q[0, :, hh] @ K[0, :, hh].T          # [queries, keys]: column j = profile of key j
        Sn = S / np.linalg.norm(S, axis=0, keepdims=True)
        assert np.max(np.abs(U[0, hh] @ U[0, hh].T - Sn.T @ Sn)) < 1e-12


def test_tree_capacities():
    # 1800 full leaves (the video grid): every leaf holds 64 tokens
    slots = rb.tree_slots(115200, 64)
    assert len(slots) == 12
    leaves = [(s, e) for (s, e, c) in slots[-1] if c == 1]
    assert len(leaves) == 1800 and all(e - s == 64 for s, e in leaves)
    # 200 tokens: 4 leaves, the last one short; children halve the leaf count
    slots = rb.tree_slots(200, 64)
    assert slots[1] == [(0, 128, 2), (128, 200, 2)]
    assert [(s, e) for (s, e, c) in slots[-1] if c == 1] == [(0, 64), (64, 128), (128, 192), (192, 200)]
    # 3 leaves: the first child takes 1 (and passes through), the second 2
    slots = rb.tree_slots(192, 64)
    assert slots[1] == [(0, 64, 1), (64, 192, 2)]
    assert slots[2] == [(0, 0, 0), (0, 64, 1), (64, 128, 1), (128, 192, 1)]


def test_principal_axis_of_landmarks():
    """With a clear leading direction the 16 power iterations give the top
    eigenvector of the centred landmark covariance."""
    rng = np.random.default_rng(52)
    n, D = 640, 10
    axis = np.zeros(D)
    axis[3] = 1.0
    U = rng.standard_normal((n, D)) * 0.1 + np.outer(rng.standard_normal(n) * 3.0, axis)
    v = rb.split_direction(U)
    ranks = [(2 * s + 1) * n // 64 for s in range(32)]
    X = U[ranks] - U[ranks].mean(axis=0)
    w, V = np.linalg.eigh(X.T @ X)
    assert abs(abs(v @ V[:, -1]) - 1.0) < 1e-9
    assert v[np.argmax(np.abs(v))] > 0


def test_centred_gram_null_space_and_ramp_start():
    """Centring puts the all-ones vector in the landmark Gram matrix's null
    space, so the iteration starts from the ramp s - 15.5, which is not."""
    rng = np.random.default_rng(57)
    X = rng.standard_normal((32, 16))
    X -= X.mean(axis=0)
    G = X @ X.T
    assert np.max(np.abs(G @ np.ones(32))) < 1e-12
    ramp = np.arange(32) - 15.5
    assert np.linalg.norm(G @ ramp) > 1.0 and abs(ramp @ ramp - 2728.0) < 1e-12


def test_interleaved_clusters_are_separated():
    """Keys of two score patterns interleaved in token order (a seeded random
    half each); the root's equal-capacity split puts each pattern in one child
    (the page's teaching experiment: interleaved tokens, concentrated after
    grouping)."""
    rng = np.random.default_rng(53)
    B, N, h, D = 1, 512, 1, 8
    Q = rng.standard_normal((B, N, h, D))
    wa, wb = rng.standard_normal(D), rng.standard_normal(D)
    in_a = np.zeros(N, dtype=bool)
    in_a[rng.permutation(N)[:N // 2]] = True
    K = np.where(in_a[None, :, None, None], wa, wb) + 0.05 * rng.standard_normal((B, N, h, D))
    U = rb.key_features(K, Q)
    orders = rb.reblock_orders(U[0, 0], 64)
    first = orders[1][:N // 2]
    assert len(set(in_a[first])) == 1  # one child holds exactly one pattern


def test_permutation_invariance_dense():
    """Reblocked layout, every block kept, outputs scattered back to their
    positions: dense attention exactly (torch SDPA, float64)."""
    rng = np.random.default_rng(54)
    B, N, h, D, M = 1, 200, 1, 8, 64
    Q, K, V = (rng.standard_normal((B, N, h, D)) for _ in range(3))
    U = rb.key_features(K, Q)
    orders = rb.reblock_orders(U[0, 0], M)
    assert np.array_equal(np.sort(orders[-1]), np.arange(N))
    perm, block_len = rb.reblock_tables(orders[-1], M)
    J = len(block_len)
    idx = np.broadcast_to(np.arange(J), (B, h, J, J)).copy()
    O, _ = oracle.vsa_attention(Q, K, V, perm, block_len, M, idx, np.full((B, h, J), J))
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(Q[0, :, 0])[None, None], torch.from_numpy(K[0, :, 0])[None, None],
        torch.from_numpy(V[0, :, 0])[None, None])[0, 0].numpy()
    assert np.max(np.abs(O[0, :, 0] - ref)) < 1e-12


def test_checker_accepts_the_rule_and_catches_swaps():
    rng = np.random.default_rng(55)
    N, D, M = 400, 6, 64
    U = rng.standard_normal((N, D))
    U /= np.linalg.norm(U, axis=1, keepdims=True)
    orders = rb.reblock_orders(U, M)
    splits, viol, flips, worst = rb.check_orders(U, orders, M, 1e-9)
    assert (splits, viol, flips) == (len([1 for lvl in rb.tree_slots(N, M)[:-1] for (s, e, c) in lvl if c > 1]), 0, 0)
    assert worst == 0.0
    # a planted swap of two far-apart positions of the root's sorted order
    # breaks the root split
    bad = [o.copy() for o in orders]
    bad[1][[0, 150]] = bad[1][[150, 0]]
    _, viol, _, _ = rb.check_orders(U, bad, M, 1e-9)
    assert viol > 0


def test_split_checker_on_oracle_directions():
    """check_splits accepts the oracle's own tree with its own directions and
    rejects a direction that is valid but not principal."""
    rng = np.random.default_rng(56)
    N, D, M = 400, 6, 64
    U = rng.standard_normal((N, D)) * np.array([3.0, 1.0, 1.0, 0.5, 0.5, 0.2])
    U /= np.linalg.norm(U, axis=1, keepdims=True)
    orders = rb.reblock_orders(U, M)
    slots = rb.tree_slots(N, M)
    dirs = []
    for li, lvl in enumerate(slots[:-1]):
        level = np.zeros((len(lvl), D))
        for si, (s, e, c) in enumerate(lvl):
            if c > 1:
                level[si] = rb.split_direction(U[orders[li][s:e]])
        dirs.append(level)
    splits, viol, inv, short = rb.check_splits(U, orders, dirs, M, 1e-12, 1e-9)
    assert viol == 0 and inv == 0.0 and short <= 1e-12 and splits > 0
    # the root's direction replaced by its least principal landmark axis
    n = N
    ranks = [(2 * t + 1) * n // 64 for t in range(32)]
    X = U[ranks] - U[ranks].mean(axis=0)
    w, V = np.linalg.eigh(X.T @ X)
    weak = V[:, 0] * np.sign(V[np.argmax(np.abs(V[:, 0])), 0])
    bad_dirs = [d.copy() for d in dirs]
    bad_dirs[0][0] = weak
    bad_orders = [o.copy() for o in orders]
    bad_orders[1] = orders[0][np.argsort(U @ weak, kind="stable")]
    _, viol, _, short = rb.check_splits(U, bad_orders, bad_dirs, M, 1e-12, 1e-3)
    assert viol >= 1 and short > 0.5
