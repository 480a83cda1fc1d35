"""3D spatio-temporal tiling and the keep budget (oracle, float64 / integer).

Source: "VSA 实现详解：三维分块、均值路由与块稀疏 Attention", section 1 (token
numbering index(t,y,x) = t*H*W + y*W + x, block count J as a product of
ceilings, true lengths of edge blocks), section 3 (pack: members of a block
become contiguous; outputs go back through the inverse map; padding outputs
are dropped) and section 2.2 (the keep budget R_r).

Readings where the page is silent:
* members inside a block are listed with t slowest and x fastest, the same
  flattening the page uses for whole tokens; the block id has its x-block index
  fastest (blocks A, B, C, D = top-left, top-right, bottom-left, bottom-right);
* an edge block keeps the same order over its valid extent, its valid members
  occupy slots 0..n-1 and the padding slots (perm = -1) sit at its end;
* the budget subtracts 1e-9 before the ceiling so that (1-0.7)*10 gives 3.
"""

import math

import numpy as np


def tile_dims(T, H, W, bT, bH, bW):
    """Return (J, M): block count and full-block capacity (section 1)."""
    for v in (T, H, W, bT, bH, bW):
        if int(v) <= 0:
            raise ValueError("grid and block sizes must be positive")
    JT = -(-T // bT)
    JH = -(-H // bH)
    JW = -(-W // bW)
    return JT * JH * JW, bT * bH * bW


def tile_index(T, H, W, bT, bH, bW):
    """Build the packing tables of the 3D tiling (sections 1 and 3).

    Returns a dict with
      perm      int64 [J*M]  token id held by packed slot p (-1 for padding)
      block_len int64 [J]    true length n_b of block b
      inv       int64 [N]    packed slot of each token (inv[perm[p]] = p)
      J, M, N
    """
    J, M = tile_dims(T, H, W, bT, bH, bW)
    JH = -(-H // bH)
    JW = -(-W // bW)
    N = T * H * W
    perm = np.full(J * M, -1, dtype=np.int64)
    block_len = np.zeros(J, dtype=np.int64)
    for b in range(J):
        bt, rem = divmod(b, JH * JW)
        by, bx = divmod(rem, JW)
        members = []
        for t in range(bt * bT, min(T, (bt + 1) * bT)):
            for y in range(by * bH, min(H, (by + 1) * bH)):
                for x in range(bx * bW, min(W, (bx + 1) * bW)):
                    members.append(t * H * W + y * W + x)
        block_len[b] = len(members)
        perm[b * M: b * M + len(members)] = members
    inv = np.full(N, -1, dtype=np.int64)
    valid = perm >= 0
    inv[perm[valid]] = np.nonzero(valid)[0]
    return {"perm": perm, "block_len": block_len, "inv": inv, "J": J, "M": M, "N": N}


def keep_budget(drop_ratio, J):
    """R = max(1, min(ceil((1 - s) * J), J)) (section 2.2), with a 1e-9 guard."""
    return max(1, min(int(math.ceil((1.0 - float(drop_ratio)) * J - 1e-9)), int(J)))
