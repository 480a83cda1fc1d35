"""Pins for the oracle's Spark-Reweight summaries and joint softmax (CPU only).

Independent references: the page's printed two-token example, torch's
scaled_dot_product_attention in float64 (dense attention), scipy's logsumexp,
closed forms (entropy of the in-block weights, the tangent bound of a convex
log-mass) and the degenerate cases where a summary must equal its block.
"""

import math

import numpy as np
import pytest
import torch
from scipy.special import logsumexp

import oracle


def _dense(q, k, v):
    """Dense attention of [n, D] queries over [m, D] keys via torch SDPA (float64)."""
    o = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None, None], torch.from_numpy(k)[None, None], torch.from_numpy(v)[None, None])
    return o[0, 0].numpy()


def _f(g, key):
    return float(g[key][0])


def test_two_token_example(golden):
    """Section 07/08 numbers: mass, mean-summary mass, values, k~, b, virtual logit."""
    g = golden("spark_reweight_two_token.txt")
    keys = np.array([float(x) for x in g["keys"]])
    vals = np.array([float(x) for x in g["values"]])
    q = _f(g, "query")
    # true mass and the mean-key summary with the count correction
    assert abs(np.exp(q * keys).sum() - _f(g, "true_mass")) < 5e-7
    assert abs(len(keys) * np.exp(q * keys.mean()) - _f(g, "mean_key_mass")) < 1e-12
    assert abs(vals.mean() - _f(g, "mean_value")) < 1e-12
    w = np.exp(q * keys) / np.exp(q * keys).sum()
    assert abs(w @ vals - _f(g, "weighted_value")) < 5e-7
    # the same block through block_summaries: one block of m = 2 tokens, d = 1
    K = keys.reshape(1, 2, 1, 1)
    V = vals.reshape(1, 2, 1, 1)
    anchor = np.full((1, 1, 1), _f(g, "anchor"))
    ks, vs, b, lm = oracle.block_summaries(K, V, [0, 1], [2], 2, anchor)
    assert abs(ks[0, 0, 0, 0] - _f(g, "summary_key")) < 5e-7
    assert abs(vs[0, 0, 0, 0] - _f(g, "summary_value")) < 5e-7
    assert abs(b[0, 0, 0] - _f(g, "bias")) < 5e-7
    z = oracle.virtual_logit(np.array([[q]]), ks[0, 0].T, b[0, 0], 1.0)[0, 0]
    assert abs(z - _f(g, "virtual_logit")) < 5e-7
    assert abs(math.exp(z) - _f(g, "true_mass")) < 5e-6
    assert abs(lm[0, 0, 0] - math.log(_f(g, "true_mass"))) < 1e-7


def _case(geom, h=2, D=8, seed=0):
    rng = np.random.default_rng(seed)
    T, H, W, bT, bH, bW = geom
    N = T * H * W
    tab = oracle.tile_index(*geom)
    K = rng.standard_normal((1, N, h, D))
    V = rng.standard_normal((1, N, h, D))
    return rng, tab, K, V


def _random_kept(rng, h, J, kmax):
    idx = np.full((1, h, J, kmax), -1, dtype=np.int64)
    num = np.zeros((1, h, J), dtype=np.int64)
    for hh in range(h):
        for i in range(J):
            n = int(rng.integers(0, kmax + 1))
            sel = np.sort(rng.choice(J, size=n, replace=False))
            idx[0, hh, i, :n] = sel
            num[0, hh, i] = n
    return idx, num


@pytest.mark.parametrize("geom", [(4, 4, 6, 2, 2, 3), (5, 3, 7, 2, 2, 4)])
def test_exact_at_anchor(geom):
    """Every query equal to the anchor: summaries reproduce each block's mass and
    content, so the mixed attention equals dense attention over all tokens."""
    rng, tab, K, V = _case(geom, seed=1)
    h, D = K.shape[2], K.shape[3]
    N = K.shape[1]
    a = rng.standard_normal((1, h, D))
    Q = np.broadcast_to(a[:, None], (1, N, h, D)).copy()
    anchor = oracle.anchor_queries(Q)
    assert np.allclose(anchor, a, atol=1e-15)
    ks, vs, b, _ = oracle.block_summaries(K, V, tab["perm"], tab["block_len"], tab["M"], anchor)
    idx, num = _random_kept(rng, h, tab["J"], min(3, tab["J"]))
    O, LSE = oracle.reweight_attention(Q, K, V, tab["perm"], tab["block_len"], tab["M"], idx, num, ks, vs, b)
    for hh in range(h):
        dense = _dense(Q[0, :, hh], K[0, :, hh], V[0, :, hh])
        assert np.max(np.abs(O[0, :, hh] - dense)) < 1e-12
        lse = logsumexp(Q[0, :, hh] @ K[0, :, hh].T / math.sqrt(D), axis=1)
        assert np.max(np.abs(LSE[0, hh] - lse)) < 1e-12


def test_bias_is_entropy_and_bounded():
    """b = -sum p log p of the in-block weights at the anchor, 0 <= b <= log n."""
    rng, tab, K, V = _case((4, 4, 6, 2, 2, 3), seed=2)
    h, D = K.shape[2], K.shape[3]
    a = 2.0 * rng.standard_normal((1, h, D))
    ks, vs, b, lm = oracle.block_summaries(K, V, tab["perm"], tab["block_len"], tab["M"], a)
    M = tab["M"]
    for hh in range(h):
        for j in range(tab["J"]):
            toks = tab["perm"][j * M: j * M + tab["block_len"][j]]
            logits = K[0, toks, hh] @ a[0, hh] / math.sqrt(D)
            p = np.exp(logits - logsumexp(logits))
            assert abs(b[0, hh, j] + (p * np.log(p)).sum()) < 1e-12
            assert -1e-12 <= b[0, hh, j] <= math.log(len(toks)) + 1e-12
            assert abs(lm[0, hh, j] - logsumexp(logits)) < 1e-12
            assert np.allclose(ks[0, hh, j], p @ K[0, toks, hh], atol=1e-13)
            assert np.allclose(vs[0, hh, j], p @ V[0, toks, hh], atol=1e-13)


def test_virtual_logit_is_tangent_lower_bound():
    """log Z_B is convex in q and the virtual logit is its tangent at a."""
    rng, tab, K, V = _case((4, 4, 6, 2, 2, 3), seed=3)
    h, D = K.shape[2], K.shape[3]
    a = rng.standard_normal((1, h, D))
    ks, vs, b, lm = oracle.block_summaries(K, V, tab["perm"], tab["block_len"], tab["M"], a)
    M = tab["M"]
    qs = 1.5 * rng.standard_normal((64, D))
    for hh in range(h):
        for j in range(tab["J"]):
            toks = tab["perm"][j * M: j * M + tab["block_len"][j]]
            true = logsumexp(qs @ K[0, toks, hh].T / math.sqrt(D), axis=1)
            z = oracle.virtual_logit(qs, ks[0, hh, j], b[0, hh, j], 1.0 / math.sqrt(D))
            assert np.all(z <= true + 1e-12)
            za = oracle.virtual_logit(a[0, hh][None], ks[0, hh, j], b[0, hh, j], 1.0 / math.sqrt(D))[0]
            assert abs(za - lm[0, hh, j]) < 1e-12


def test_all_blocks_kept_is_the_exact_path():
    """With every block kept there is no virtual token: plain VSA attention."""
    rng, tab, K, V = _case((5, 3, 7, 2, 2, 4), seed=4)
    h, J = K.shape[2], tab["J"]
    Q = rng.standard_normal(K.shape)
    idx = np.broadcast_to(np.arange(J), (1, h, J, J)).copy()
    num = np.full((1, h, J), J)
    ks, vs, b, _ = oracle.block_summaries(K, V, tab["perm"], tab["block_len"], tab["M"], oracle.anchor_queries(Q))
    O1, L1 = oracle.reweight_attention(Q, K, V, tab["perm"], tab["block_len"], tab["M"], idx, num, ks, vs, b)
    O2, L2 = oracle.vsa_attention(Q, K, V, tab["perm"], tab["block_len"], tab["M"], idx, num)
    assert np.max(np.abs(O1 - O2)) < 1e-13
    assert np.max(np.abs(L1 - L2)) < 1e-13


def test_single_token_blocks_equal_dense():
    """Blocks of one token: the summary is the token itself (p = 1, b = 0), so any
    kept set gives dense attention."""
    rng, tab, K, V = _case((3, 4, 5, 1, 1, 1), seed=5)
    h, D, N, J = K.shape[2], K.shape[3], K.shape[1], tab["J"]
    Q = rng.standard_normal(K.shape)
    ks, vs, b, _ = oracle.block_summaries(K, V, tab["perm"], tab["block_len"], tab["M"], oracle.anchor_queries(Q))
    assert np.max(np.abs(b)) < 1e-15
    idx, num = _random_kept(rng, h, J, 7)
    O, _ = oracle.reweight_attention(Q, K, V, tab["perm"], tab["block_len"], tab["M"], idx, num, ks, vs, b)
    for hh in range(h):
        assert np.max(np.abs(O[0, :, hh] - _dense(Q[0, :, hh], K[0, :, hh], V[0, :, hh]))) < 1e-12


def test_mean_summary_differs_from_reweight():
    """The plain mean summary (mean key, mean value, + log n) is not exact at the
    anchor while the reweighted one is; a guard against the oracle silently
    using means."""
    rng, tab, K, V = _case((4, 4, 6, 2, 2, 3), seed=6)
    h, D, N, J, M = K.shape[2], K.shape[3], K.shape[1], tab["J"], tab["M"]
    a = rng.standard_normal((1, h, D))
    Q = np.broadcast_to(a[:, None], (1, N, h, D)).copy()
    mk = np.zeros((1, h, J, D)); mv = np.zeros((1, h, J, D)); mb = np.zeros((1, h, J))
    for j in range(J):
        toks = tab["perm"][j * M: j * M + tab["block_len"][j]]
        mk[0, :, j] = K[0, toks].mean(axis=0)
        mv[0, :, j] = V[0, toks].mean(axis=0)
        mb[0, :, j] = math.log(len(toks))
    idx = np.full((1, h, J, 1), -1); num = np.zeros((1, h, J), dtype=np.int64)
    O, _ = oracle.reweight_attention(Q, K, V, tab["perm"], tab["block_len"], M, idx, num, mk, mv, mb)
    dense = _dense(Q[0, :, 0], K[0, :, 0], V[0, :, 0])
    assert np.max(np.abs(O[0, :, 0] - dense)) > 1e-3


def test_seeded_construction_of_section_10(golden):
    """The page's own check (section 10): with the summaries taken at the
    query, the mixed softmax reproduces dense attention to rounding; plain
    mean summaries miss it by the printed 0.240925."""
    g = golden("spark_seeded_construction.txt")
    n, dk, dv, blk = (int(g[key][0]) for key in ("tokens", "key_dim", "value_dim", "block"))
    rng = np.random.default_rng(int(g["seed"][0]))
    k = rng.normal(size=(n, dk))
    v = rng.normal(size=(n, dv))
    a = rng.normal(size=dk)
    tab = oracle.tile_index(n, 1, 1, blk, 1, 1)
    J, M = tab["J"], tab["M"]
    # the value channels are padded with zeros up to the key width (the
    # oracle keeps one channel count); the padding channels stay zero
    K = k.reshape(1, n, 1, dk)
    V = np.zeros((1, n, 1, dk))
    V[0, :, 0, :dv] = v
    Q = np.broadcast_to(a, (1, n, 1, dk)).copy()  # every query row is a
    exact = [int(x) for x in g["exact_blocks"]]
    idx = np.full((1, 1, J, len(exact)), -1, dtype=np.int64)
    idx[0, 0, :, :] = exact
    num = np.full((1, 1, J), len(exact), dtype=np.int64)
    dense = _dense(a[None], k, v)[0]
    ks, vs, b, _ = oracle.block_summaries(K, V, tab["perm"], tab["block_len"], M, a.reshape(1, 1, dk))
    O, _ = oracle.reweight_attention(Q, K, V, tab["perm"], tab["block_len"], M, idx, num, ks, vs, b)
    err = np.abs(O[0, :, 0, :dv] - dense).max()
    assert err <= float(g["reweight_assert"][0])
    assert np.all(O[0, :, 0, dv:] == 0.0)
    mk = np.zeros_like(ks)
    mv = np.zeros_like(vs)
    for j in range(J):
        toks = tab["perm"][j * M: (j + 1) * M]
        mk[0, 0, j] = K[0, toks, 0].mean(axis=0)
        mv[0, 0, j] = V[0, toks, 0].mean(axis=0)
    mb = np.full((1, 1, J), math.log(M))
    Om, _ = oracle.reweight_attention(Q, K, V, tab["perm"], tab["block_len"], M, idx, num, mk, mv, mb)
    err_mean = np.abs(Om[0, :, 0, :dv] - dense).max()
    assert abs(err_mean - float(g["mean_summary_max_err"][0])) <= 5e-7
