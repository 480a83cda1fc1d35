"""H3 multi-region layout and grouped routing (oracle, float64).

TEST INFRASTRUCTURE ONLY (see the package docstring).

Source: "VSA 实现详解：三维分块、均值路由与块稀疏 Attention", section 5.2 (the
layout) and section 5.3 (the default "exempt" routing).

Layout: the caller lists the segments of the packed sequence in their original
order; a dense segment (text, reference image, audio) is a token count, a
video region is a (T, H, W) grid.  Every dense segment is cut on its own into
consecutive 1D chunks of the block capacity M (its last chunk is padded, no
chunk mixes two segments); all dense chunks come first, in segment order, and
form the prefix; the video regions follow in their order, each cut into 3D
blocks of (bT, bH, bW) = M tokens exactly as a single video is (section 1).
Every block keeps its true length; outputs go back to the original positions.

Routing: one score matrix E = Q_bar K_bar^T / sqrt(D) over all blocks.  A
prefix (context) query block keeps every block.  A video query block keeps
every prefix block and, in each video region r separately, the TopK of its
scores restricted to that region's blocks with the region's own budget R_r;
the kept set is the union (one softmax over it, as in section 4).
"""

import numpy as np

from .routing import routing_matrix, select_topk
from .tiling import tile_index


def h3_layout(segments, block):
    """Tables of a multi-region layout.

    segments: list of ints (dense segment of that many tokens) and (T, H, W)
    tuples (video regions), in the order of the original sequence.
    block: (bT, bH, bW); the block capacity M = bT*bH*bW applies to dense
    chunks too.

    Returns a dict: perm int64 [J*M] (original positions, -1 padding), block_len
    [J], inv [N] (packed slot of every original position), J, M, N,
    num_prefix, spans (half-open block ranges of the video regions, in order),
    segment_of_block [J].
    """
    bT, bH, bW = block
    M = bT * bH * bW
    lengths, offsets, off = [], [], 0
    for s in segments:
        n = int(s) if np.isscalar(s) else int(s[0]) * int(s[1]) * int(s[2])
        if n < 0 or (not np.isscalar(s) and n == 0):
            raise ValueError("bad segment %r" % (s,))
        lengths.append(n)
        offsets.append(off)
        off += n
    N = off
    perm, block_len, seg_of = [], [], []
    # prefix: the dense segments' chunks, in segment order
    for si, s in enumerate(segments):
        if not np.isscalar(s):
            continue
        n = lengths[si]
        for c0 in range(0, n, M):
            cnt = min(M, n - c0)
            perm.extend(offsets[si] + c0 + r for r in range(cnt))
            perm.extend([-1] * (M - cnt))
            block_len.append(cnt)
            seg_of.append(si)
    num_prefix = len(block_len)
    spans = []
    for si, s in enumerate(segments):
        if np.isscalar(s):
            continue
        T, H, W = (int(v) for v in s)
        tab = tile_index(T, H, W, bT, bH, bW)
        b0 = len(block_len)
        p = np.asarray(tab["perm"])
        perm.extend(np.where(p >= 0, p + offsets[si], -1).tolist())
        block_len.extend(int(v) for v in tab["block_len"])
        seg_of.extend([si] * tab["J"])
        spans.append((b0, len(block_len)))
    perm = np.asarray(perm, dtype=np.int64)
    J = len(block_len)
    inv = np.full(N, -1, dtype=np.int64)
    valid = np.nonzero(perm >= 0)[0]
    inv[perm[valid]] = valid
    return {"perm": perm, "block_len": np.asarray(block_len, dtype=np.int64), "inv": inv, "J": J, "M": M,
            "N": N, "num_prefix": num_prefix, "spans": spans,
            "segment_of_block": np.asarray(seg_of, dtype=np.int64)}


def h3_route(qbar, kbar, num_prefix, spans, budgets, kmax=None):
    """Grouped (exempt) routing.

    qbar, kbar: [B, h, J, D] pooled means over the layout's blocks.
    budgets: R_r per video region (1 <= R_r <= the region's block count).
    Returns q2k_idx [B, h, J, kmax] (ascending, -1 fill; kmax defaults to J),
    q2k_num [B, h, J], and gap [B, h, J, regions]: for video rows, the score
    difference between the R_r-th and (R_r+1)-th block of each region (+inf
    when the region is kept whole), for near-tie exemption; context rows +inf.
    """
    E = routing_matrix(qbar, kbar)
    B, h, J, _ = E.shape
    kmax = J if kmax is None else int(kmax)
    if len(budgets) != len(spans):
        raise ValueError("one budget per video region")
    idx = np.full((B, h, J, kmax), -1, dtype=np.int64)
    num = np.zeros((B, h, J), dtype=np.int64)
    gap = np.full((B, h, J, max(1, len(spans))), np.inf)
    picks = []
    for r, (b0, b1) in enumerate(spans):
        R = int(budgets[r])
        if not 1 <= R <= b1 - b0:
            raise ValueError("budget %d outside [1, %d]" % (R, b1 - b0))
        sel, _, g = select_topk(E[:, :, :, b0:b1], R)
        picks.append(sel[..., :R] + b0)
        gap[..., r] = g
    for b in range(B):
        for hh in range(h):
            for i in range(J):
                if i < num_prefix:
                    row = np.arange(J)
                    gap[b, hh, i, :] = np.inf
                else:
                    row = np.concatenate([np.arange(num_prefix)] + [pk[b, hh, i] for pk in picks])
                    row = np.sort(row)
                if len(row) > kmax:
                    raise ValueError("kmax %d < %d kept blocks" % (kmax, len(row)))
                idx[b, hh, i, :len(row)] = row
                num[b, hh, i] = len(row)
    return idx, num, gap
