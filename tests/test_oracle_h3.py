"""Pins for the oracle's H3 multi-region layout and grouped routing (CPU only).

Independent references: the page's printed metadata and block counts
(tests/golden/h3_layout_example.txt), block membership recomputed from token
coordinates, a crafted score pattern for the per-region quota, and torch's
scaled_dot_product_attention in float64 with a token-level mask for the one
softmax over the union of kept blocks.
"""

import numpy as np
import torch

import oracle

# Segments of the page's example: text 130, reference video, image 60, audio
# 200, target video (grids chosen to give the printed 4 and 8 full blocks of
# 128; the page does not print the grids).
PAGE_SEGMENTS = [130, (2, 16, 16), 60, 200, (4, 16, 16)]
PAGE_BLOCK = (2, 8, 8)


def _ints(g, key):
    return [int(v) for v in g[key]]


def test_page_example_layout(golden):
    g = golden("h3_layout_example.txt")
    lay = oracle.h3_layout(PAGE_SEGMENTS, PAGE_BLOCK)
    assert lay["num_prefix"] == _ints(g, "num_prefix_tiles")[0]
    sp = _ints(g, "video_tile_spans")
    assert lay["spans"] == [(sp[0], sp[1]), (sp[2], sp[3])]
    head = _ints(g, "block_sizes_head")
    assert list(lay["block_len"][:len(head)]) == head
    assert (lay["block_len"][len(head):] == 128).all()
    assert lay["J"] == _ints(g, "num_blocks")[0]
    assert lay["N"] == int(lay["block_len"].sum()) == _ints(g, "valid_length")[0]
    assert lay["J"] * lay["M"] == _ints(g, "tiled_length")[0]


def test_page_example_counts(golden):
    g = golden("h3_layout_example.txt")
    lay = oracle.h3_layout(PAGE_SEGMENTS, PAGE_BLOCK)
    keep = float(g["keep_ratio"][0])
    budgets = [oracle.keep_budget(1.0 - keep, b1 - b0) for b0, b1 in lay["spans"]]
    assert budgets == [1, 2]
    rng = np.random.default_rng(40)
    qbar = rng.standard_normal((1, 2, lay["J"], 16))
    kbar = rng.standard_normal((1, 2, lay["J"], 16))
    idx, num, _ = oracle.h3_route(qbar, kbar, lay["num_prefix"], lay["spans"], budgets)
    P = lay["num_prefix"]
    assert (num[:, :, :P] == _ints(g, "blocks_per_context_row")[0]).all()
    assert (num[:, :, P:] == _ints(g, "blocks_per_video_row")[0]).all()
    # every video row holds the whole prefix, then ascending ids
    assert (idx[:, :, P:, :P] == np.arange(P)).all()
    kept = idx[:, :, :, :8]
    assert (np.diff(kept, axis=-1) > 0).all()


def test_r2v_figure_counts(golden):
    """Two context blocks, reference videos of 3 blocks each, an output video
    of 4 blocks, budgets 1/3, 1/3, 2/4: 6 blocks per video row."""
    g = golden("h3_layout_example.txt")
    # capacity 4 (1x2x2): 8 dense tokens = 2 blocks; (1,2,6) = 3 blocks; (1,4,4) = 4 blocks
    lay = oracle.h3_layout([8, (1, 2, 6), (1, 2, 6), (1, 4, 4)], (1, 2, 2))
    assert lay["num_prefix"] == _ints(g, "r2v_context_blocks")[0]
    assert [b1 - b0 for b0, b1 in lay["spans"]] == _ints(g, "r2v_region_blocks")
    rng = np.random.default_rng(41)
    qbar = rng.standard_normal((1, 1, lay["J"], 8))
    kbar = rng.standard_normal((1, 1, lay["J"], 8))
    idx, num, _ = oracle.h3_route(qbar, kbar, lay["num_prefix"], lay["spans"], _ints(g, "r2v_budgets"))
    P = lay["num_prefix"]
    assert (num[0, 0, P:] == _ints(g, "r2v_blocks_per_video_row")[0]).all()
    assert (num[0, 0, :P] == lay["J"]).all()


def test_quota_is_per_region():
    """Output-video keys score far above the reference keys for every query,
    yet each region keeps its own budget: the reference quota is not taken
    by the output video (a single TopK over both regions would take none of it)."""
    lay = oracle.h3_layout([6, (1, 4, 8), (2, 4, 8)], (1, 2, 2))
    J, P = lay["J"], lay["num_prefix"]
    (r0, r1), (o0, o1) = lay["spans"]
    rng = np.random.default_rng(42)
    D = 4
    qbar = np.zeros((1, 1, J, D))
    qbar[..., 0] = 1.0
    qbar[..., 1:] = 0.01 * rng.standard_normal((1, 1, J, D - 1))
    kbar = rng.standard_normal((1, 1, J, D)) * 0.1
    kbar[0, 0, o0:o1, 0] += 10.0  # output-video blocks dominate every row
    budgets = [2, 3]
    idx, num, _ = oracle.h3_route(qbar, kbar, P, lay["spans"], budgets)
    E = oracle.routing_matrix(qbar, kbar)
    for i in range(P, J):
        row = idx[0, 0, i, :num[0, 0, i]]
        ref = row[(row >= r0) & (row < r1)]
        out = row[(row >= o0) & (row < o1)]
        assert len(ref) == 2 and len(out) == 3
        # within a region: exactly the highest scores
        assert set(ref) == set(r0 + np.argsort(-E[0, 0, i, r0:r1], kind="stable")[:2])
        assert set(out) == set(o0 + np.argsort(-E[0, 0, i, o0:o1], kind="stable")[:3])
        # a single TopK of 5 over both regions keeps no reference block
        glob = np.argsort(-E[0, 0, i, r0:o1], kind="stable")[:5] + r0
        assert not ((glob >= r0) & (glob < r1)).any()


def _block_of_token(segments, block):
    """Layout block of every original position, from coordinates alone."""
    bT, bH, bW = block
    M = bT * bH * bW
    sizes, starts, off = [], [], 0
    for s in segments:
        n = int(s) if np.isscalar(s) else int(np.prod(s))
        sizes.append(n)
        starts.append(off)
        off += n
    out = np.full(off, -1)
    nb = 0
    for si, s in enumerate(segments):
        if np.isscalar(s):
            for u in range(sizes[si]):
                out[starts[si] + u] = nb + u // M
            nb += -(-sizes[si] // M)
    for si, s in enumerate(segments):
        if np.isscalar(s):
            continue
        T, H, W = s
        JH, JW = -(-H // bH), -(-W // bW)
        for t in range(T):
            for y in range(H):
                for x in range(W):
                    out[starts[si] + (t * H + y) * W + x] = nb + ((t // bT) * JH + y // bH) * JW + x // bW
        nb += -(-T // bT) * JH * JW
    return out


def test_layout_brute_force():
    segments = [5, (3, 5, 6), 9, (2, 3, 3), 1, (5, 4, 2)]
    block = (2, 2, 2)
    lay = oracle.h3_layout(segments, block)
    M = lay["M"]
    bo = _block_of_token(segments, block)
    assert lay["N"] == len(bo)
    perm, bl = lay["perm"], lay["block_len"]
    # every position once; padding only after the valid members
    valid = perm[perm >= 0]
    assert np.array_equal(np.sort(valid), np.arange(lay["N"]))
    for b in range(lay["J"]):
        row = perm[b * M:(b + 1) * M]
        assert (row[:bl[b]] >= 0).all() and (row[bl[b]:] == -1).all()
        assert (bo[row[:bl[b]]] == b).all()
    assert np.array_equal(lay["inv"] // M, bo)
    # prefix blocks: 1 + 2 + 1 chunks of three dense segments
    assert lay["num_prefix"] == 4
    assert lay["spans"] == [(4, 4 + 2 * 3 * 3), (22, 22 + 4), (26, 26 + 3 * 2)]


def test_union_softmax_is_masked_dense():
    """Attention over a grouped-routing table = one softmax over the kept
    tokens: dense SDPA with a token mask from coordinates (context queries
    see every key)."""
    segments = [7, (2, 4, 4), 3, (3, 4, 6)]
    block = (1, 2, 4)
    lay = oracle.h3_layout(segments, block)
    rng = np.random.default_rng(43)
    B, h, D = 1, 2, 8
    N = lay["N"]
    Q, K, V = (rng.standard_normal((B, N, h, D)) for _ in range(3))
    qbar = oracle.pool_blocks(Q, lay["perm"], lay["block_len"], lay["M"])
    kbar = oracle.pool_blocks(K, lay["perm"], lay["block_len"], lay["M"])
    budgets = [2, 3]
    idx, num, _ = oracle.h3_route(qbar, kbar, lay["num_prefix"], lay["spans"], budgets)
    O, _ = oracle.vsa_attention(Q, K, V, lay["perm"], lay["block_len"], lay["M"], idx, num)
    bo = _block_of_token(segments, block)
    for hh in range(h):
        allowed = np.zeros((N, N), dtype=bool)
        for qt in range(N):
            kept = set(idx[0, hh, bo[qt], :num[0, hh, bo[qt]]].tolist())
            allowed[qt] = np.isin(bo, list(kept))
        assert allowed[bo < lay["num_prefix"]].all()  # context queries are dense
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(Q[0, :, hh])[None, None], torch.from_numpy(K[0, :, hh])[None, None],
            torch.from_numpy(V[0, :, hh])[None, None], attn_mask=torch.from_numpy(allowed)[None, None])[0, 0]
        assert np.max(np.abs(O[0, :, hh] - ref.numpy())) < 1e-12
