"""Pins for the oracle's VSA, NSA and KV-outer attention (CPU only).

Independent references: torch's scaled_dot_product_attention in float64 on
the CPU (a library routine), token masks built by brute force from token
coordinates, scipy's logsumexp, and the page's own per-token NSA loop
re-done step by step.
"""

import math

import numpy as np
import pytest
import torch
from scipy.special import logsumexp

import oracle


def _sdpa(q, k, v, mask=None, causal=False):
    """Reference attention via torch SDPA, float64, [N, h, D] numpy arrays."""
    tq = torch.from_numpy(np.ascontiguousarray(q.transpose(1, 0, 2)))[None]
    tk = torch.from_numpy(np.ascontiguousarray(k.transpose(1, 0, 2)))[None]
    tv = torch.from_numpy(np.ascontiguousarray(v.transpose(1, 0, 2)))[None]
    m = None if mask is None else torch.from_numpy(mask)
    o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=m, is_causal=causal)
    return o[0].numpy().transpose(1, 0, 2)


def _block_of(geom):
    T, H, W, bT, bH, bW = geom
    JH, JW = -(-H // bH), -(-W // bW)
    out = []
    for tok in range(T * H * W):
        t, rem = divmod(tok, H * W)
        y, x = divmod(rem, W)
        out.append(((t // bT) * JH + y // bH) * JW + x // bW)
    return np.array(out)


@pytest.mark.parametrize("geom", [(5, 3, 4, 4, 2, 2), (4, 4, 4, 4, 2, 2), (6, 5, 7, 4, 4, 4)])
def test_full_keep_equals_dense(geom):
    rng = np.random.default_rng(11)
    T, H, W = geom[:3]
    N, h, D = T * H * W, 3, 8
    Q, K, V = (rng.standard_normal((1, N, h, D)) for _ in range(3))
    tab = oracle.tile_index(*geom)
    J = tab["J"]
    idx = np.tile(np.arange(J), (1, h, J, 1))
    num = np.full((1, h, J), J)
    O, LSE = oracle.vsa_attention(Q, K, V, tab["perm"], tab["block_len"], tab["M"], idx, num)
    ref = _sdpa(Q[0], K[0], V[0])
    assert np.abs(O[0] - ref).max() < 1e-12
    logits = np.einsum("nhd,mhd->hnm", Q[0], K[0]) / math.sqrt(D)
    assert np.abs(LSE[0] - logsumexp(logits, axis=-1)).max() < 1e-12


@pytest.mark.parametrize("geom,R", [((5, 3, 4, 4, 2, 2), 3), ((4, 4, 4, 4, 2, 2), 2), ((6, 5, 7, 4, 4, 4), 3)])
def test_sparse_equals_masked_dense(geom, R):
    """Pack -> select -> attend equals masked attention in the original order."""
    rng = np.random.default_rng(12)
    T, H, W = geom[:3]
    N, h, D = T * H * W, 2, 8
    Q, K, V = (rng.standard_normal((1, N, h, D)) for _ in range(3))
    tab = oracle.tile_index(*geom)
    J, M = tab["J"], tab["M"]
    qbar = oracle.pool_blocks(Q, tab["perm"], tab["block_len"], M)
    kbar = oracle.pool_blocks(K, tab["perm"], tab["block_len"], M)
    idx, num, _ = oracle.select_topk(oracle.routing_matrix(qbar, kbar), R, kmax=J)
    O, _ = oracle.vsa_attention(Q, K, V, tab["perm"], tab["block_len"], M, idx, num)
    blk = _block_of(geom)
    for hh in range(h):
        sel = np.zeros((J, J), dtype=bool)
        for i in range(J):
            sel[i, idx[0, hh, i, :R]] = True
        mask = sel[blk[:, None], blk[None, :]]          # [N, N] token mask
        ref = _sdpa(Q[0, :, hh:hh + 1], K[0, :, hh:hh + 1], V[0, :, hh:hh + 1], mask=mask)
        assert np.abs(O[0, :, hh] - ref[:, 0]).max() < 1e-12


def test_teaching_grid_pair_count(golden):
    """J*R*M^2 allowed query-key pairs for the teaching grid at R=2."""
    g = golden("vsa_topk_example.txt")
    tab = oracle.tile_index(4, 4, 4, 4, 2, 2)
    rng = np.random.default_rng(5)
    Q, K = (rng.standard_normal((1, 64, 1, 4)) for _ in range(2))
    qbar = oracle.pool_blocks(Q, tab["perm"], tab["block_len"], 16)
    kbar = oracle.pool_blocks(K, tab["perm"], tab["block_len"], 16)
    idx, num, _ = oracle.select_topk(oracle.routing_matrix(qbar, kbar), 2)
    blk = _block_of((4, 4, 4, 4, 2, 2))
    sel = np.zeros((4, 4), dtype=bool)
    for i in range(4):
        sel[i, idx[0, 0, i]] = True
    assert sel[blk[:, None], blk[None, :]].sum() == int(g["pairs_sparse"][0])
    assert 64 * 64 == int(g["pairs_dense"][0]) and 4 * 4 == int(g["pairs_routing"][0])


def test_permutation_invariance_dense():
    """Permute Q; permute K and V with one shared permutation; restore Q order."""
    rng = np.random.default_rng(13)
    geom = (5, 3, 4, 4, 2, 2)
    N, h, D = 60, 2, 6
    Q, K, V = (rng.standard_normal((1, N, h, D)) for _ in range(3))
    tab = oracle.tile_index(*geom)
    J = tab["J"]
    idx = np.tile(np.arange(J), (1, h, J, 1))
    num = np.full((1, h, J), J)
    args = (tab["perm"], tab["block_len"], tab["M"], idx, num)
    O, _ = oracle.vsa_attention(Q, K, V, *args)
    pq, pk = rng.permutation(N), rng.permutation(N)
    O2, _ = oracle.vsa_attention(Q[:, pq], K[:, pk], V[:, pk], *args)
    restored = np.empty_like(O2)
    restored[:, pq] = O2
    assert np.abs(restored - O).max() < 1e-12
    # binding K and V to different permutations changes the result
    O3, _ = oracle.vsa_attention(Q, K[:, pk], V, *args)
    assert np.abs(O3 - O).max() > 1e-3


def test_empty_row_gives_zero():
    rng = np.random.default_rng(1)
    tab = oracle.tile_index(4, 4, 4, 4, 2, 2)
    Q, K, V = (rng.standard_normal((1, 64, 1, 4)) for _ in range(3))
    idx = np.array([[[[1, -1], [-1, -1], [0, 3], [2, 2]]]])
    num = np.array([[[1, 0, 2, 2]]])
    O, LSE = oracle.vsa_attention(Q, K, V, tab["perm"], tab["block_len"], 16, idx, num)
    rows_B = tab["perm"][16:32]
    assert (O[0, rows_B] == 0).all() and np.isneginf(LSE[0, 0, rows_B]).all()
    assert np.isfinite(O).all()


# ---------------------------------------------------------------- NSA mode

def _nsa_inputs(T, HQ, H, D, BS, S, seed):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((1, T, HQ, D))
    k = rng.standard_normal((1, T, H, D))
    v = rng.standard_normal((1, T, H, D))
    NB = -(-T // BS)
    idx = np.full((1, T, H, S), -1, dtype=np.int64)
    cnt = np.zeros((1, T, H), dtype=np.int64)
    for t in range(T):
        for r in range(H):
            cur = t // BS
            c = min(int(rng.integers(1, S + 1)), cur + 1)
            others = rng.choice(cur, size=c - 1, replace=False) if c > 1 else []
            row = sorted([cur, *others])
            idx[0, t, r, :c] = row
            cnt[0, t, r] = c
    return q, k, v, idx, cnt, NB


def _page_loop_nsa(q, k, v, block_indices, block_counts, BS):
    """The page's per-token definition, step by step, in NumPy float64."""
    B, T, HQ, D = q.shape
    H = k.shape[2]
    G = HQ // H
    S = block_indices.shape[-1]
    scale = D ** -0.5
    kk = np.repeat(k, G, axis=2)                     # heads h -> (h g)
    vv = np.repeat(v, G, axis=2)
    bi = np.repeat(block_indices, G, axis=2)
    bc = np.repeat(block_counts, G, axis=2)
    c = np.repeat(np.arange(S), BS)                  # slot of each selected token
    o = np.zeros_like(q)
    for b in range(B):
        tok = bi[b][..., None] * BS + np.arange(BS)  # [T, HQ, S, BS]
        tok = tok.reshape(T, HQ, S * BS)
        for t in range(T):
            for hq in range(HQ):
                ids = tok[t, hq]
                attn = np.full(S * BS, -np.inf)
                ok = ~((ids > t) | (c >= bc[b, t, hq]))
                attn[ok] = kk[b, ids[ok], hq] @ (q[b, t, hq] * scale)
                w = np.exp(attn - attn.max())
                w /= w.sum()
                o[b, t, hq] = w[ok] @ vv[b, ids[ok], hq]
    return o


def test_nsa_matches_page_loop():
    q, k, v, idx, cnt, _ = _nsa_inputs(T=200, HQ=8, H=2, D=8, BS=16, S=5, seed=21)
    o, _ = oracle.nsa_attention(q, k, v, idx, cnt, BS=16, causal=True)
    ref = _page_loop_nsa(q, k, v, idx, cnt, 16)
    assert np.abs(o - ref).max() < 1e-12


def test_nsa_all_visible_is_causal_dense():
    T, HQ, H, D, BS = 96, 4, 2, 8, 16
    rng = np.random.default_rng(22)
    q = rng.standard_normal((1, T, HQ, D))
    k = rng.standard_normal((1, T, H, D))
    v = rng.standard_normal((1, T, H, D))
    NB = T // BS
    idx = np.full((1, T, H, NB), -1)
    cnt = np.zeros((1, T, H), dtype=np.int64)
    for t in range(T):
        idx[0, t, :, : t // BS + 1] = np.arange(t // BS + 1)
        cnt[0, t, :] = t // BS + 1
    o, lse = oracle.nsa_attention(q, k, v, idx, cnt, BS, causal=True)
    G = HQ // H
    ref = _sdpa(q[0], np.repeat(k[0], G, axis=1), np.repeat(v[0], G, axis=1), causal=True)
    assert np.abs(o[0] - ref).max() < 1e-12


def test_nsa_local_block_only():
    T, HQ, H, D, BS = 80, 4, 1, 8, 16
    rng = np.random.default_rng(23)
    q = rng.standard_normal((1, T, HQ, D))
    k = rng.standard_normal((1, T, H, D))
    v = rng.standard_normal((1, T, H, D))
    idx = (np.arange(T) // BS)[None, :, None, None].repeat(H, 2)
    cnt = np.ones((1, T, H), dtype=np.int64)
    o, _ = oracle.nsa_attention(q, k, v, idx, cnt, BS, causal=True)
    pos = np.arange(T)
    mask = (pos[:, None] // BS == pos[None, :] // BS) & (pos[None, :] <= pos[:, None])
    ref = _sdpa(q[0], np.repeat(k[0], HQ, axis=1), np.repeat(v[0], HQ, axis=1), mask=mask)
    assert np.abs(o[0] - ref).max() < 1e-12


def test_nsa_padding_inside_count_is_skipped():
    """Reading: an entry counts only if its slot is below the count and its id >= 0."""
    q, k, v, idx, cnt, _ = _nsa_inputs(T=64, HQ=2, H=1, D=4, BS=16, S=4, seed=24)
    idx2 = idx.copy()
    cnt2 = cnt.copy()
    t = 50
    row = idx[0, t, 0, : cnt[0, t, 0]].tolist()
    idx2[0, t, 0, :] = -1
    idx2[0, t, 0, 0] = -1
    idx2[0, t, 0, 1: 1 + len(row)] = row
    cnt2[0, t, 0] = len(row) + 1
    o, _ = oracle.nsa_attention(q, k, v, idx, cnt, 16, tokens=[(0, t)])
    o2, _ = oracle.nsa_attention(q, k, v, idx2, cnt2, 16, tokens=[(0, t)])
    assert np.abs(o[0, t] - o2[0, t]).max() == 0.0


# ------------------------------------------------------------- KV-outer

def test_kvouter_combine_equals_global_softmax():
    q, k, v, idx, cnt, _ = _nsa_inputs(T=300, HQ=8, H=2, D=8, BS=32, S=6, seed=31)
    O_buf, L_buf, nslot = oracle.kvouter_partials(q, k, v, idx, BK=32, causal=True, q2k_cnt=cnt)
    O, L = oracle.lse_combine(O_buf, L_buf, nslot, G=4)
    ref, ref_lse = oracle.nsa_attention(q, k, v, idx, cnt, BS=32, causal=True)
    assert np.abs(O - ref).max() < 1e-12
    assert np.abs(L - ref_lse).max() < 1e-12
    assert (nslot == cnt).all()


def test_kvouter_slot_rule_and_partials():
    """Slot s holds the s-th smallest selected block; L_s is its log-sum-exp."""
    T, HQ, H, D, BK = 128, 4, 1, 8, 16
    rng = np.random.default_rng(32)
    q = rng.standard_normal((1, T, HQ, D))
    k = rng.standard_normal((1, T, H, D))
    v = rng.standard_normal((1, T, H, D))
    i = 100
    row = np.array([[[6, 0, -1, 3]]])                 # unsorted, with a -1
    q2k = np.full((1, T, H, 4), -1)
    q2k[0, i] = row[0]
    O_buf, L_buf, nslot = oracle.kvouter_partials(q, k, v, q2k, BK, positions=[(0, i)])
    assert nslot[0, 0] == 3
    for s, blk in enumerate([0, 3, 6]):
        keys = np.arange(blk * BK, min((blk + 1) * BK, i + 1))
        logits = q[0, i] @ k[0, keys, 0].T / math.sqrt(D)      # [HQ, n]
        lse = logsumexp(logits, axis=-1)
        w = np.exp(logits - lse[:, None])
        assert np.abs(L_buf[0, s] - lse).max() < 1e-12
        assert np.abs(O_buf[0, s] - w @ v[0, keys, 0]).max() < 1e-12
    assert np.isneginf(L_buf[0, 3]).all() and (O_buf[0, 3] == 0).all()
    # the compact rows equal the full-layout rows
    O_f, L_f, n_f = oracle.kvouter_partials(q, k, v, q2k, BK)
    assert np.array_equal(O_f[0, :, i], O_buf[0]) and np.array_equal(L_f[0, :, i], L_buf[0])
    assert np.array_equal(n_f[0, i], nslot[0])


def test_combine_single_slot_and_weights():
    rng = np.random.default_rng(33)
    O_buf = rng.standard_normal((1, 3, 5, 4, 6))
    L_buf = rng.standard_normal((1, 3, 5, 4))
    one = np.ones((1, 5, 2), dtype=np.int64)
    O, L = oracle.lse_combine(O_buf, L_buf, one, G=2)
    assert np.array_equal(O, O_buf[:, 0]) and np.array_equal(L, L_buf[:, 0])
    three = np.full((1, 5, 2), 3)
    O, L = oracle.lse_combine(O_buf, L_buf, three, G=2)
    w = np.exp(L_buf - L[:, None])
    assert np.abs(w.sum(axis=1) - 1.0).max() < 1e-14
    assert np.abs(L - logsumexp(L_buf, axis=1)).max() < 1e-14
    zero = np.zeros((1, 5, 2), dtype=np.int64)
    O, L = oracle.lse_combine(O_buf, L_buf, zero, G=2)
    assert (O == 0).all() and np.isneginf(L).all()
