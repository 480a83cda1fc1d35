"""Mean pooling, routing matrix and TopK selection (oracle, float64).

Source: "VSA 实现详解：三维分块、均值路由与块稀疏 Attention",
* section 2.1: q_bar_i = (1/n_i) * sum over the members of block i of q_a, per
  batch and head; heads and channels are never mixed; the divisor is the true
  block length n_i (section 1 for edge blocks);
* section 2.2: E = Q_bar K_bar^T / sqrt(D), shape [B, h, J, J]; each head and
  each query block selects its own TopK independently, directly on the logits;
* section 4: the index table lists the kept block ids in increasing order,
  fills the rest of the row with -1 and records the count separately.

Tie rule (the page is silent): among equal scores the lower block index wins.
The oracle also reports, per row, the gap between the R-th and (R+1)-th
largest score so that a comparison can exempt near-ties.
"""

import numpy as np


def pool_blocks(X, perm, block_len, M):
    """Per-block mean of X over each block's valid members.

    X: float array [B, N, h, D] in token order.  Returns float64 [B, h, J, D].
    """
    X = np.asarray(X, dtype=np.float64)
    B, N, h, D = X.shape
    J = len(block_len)
    out = np.zeros((B, h, J, D), dtype=np.float64)
    for i in range(J):
        n = int(block_len[i])
        if n <= 0:
            raise ValueError("every block must hold at least one token")
        members = np.asarray(perm[i * M: i * M + n])
        # sum in float64, divide by the true length
        out[:, :, i, :] = X[:, members, :, :].sum(axis=1) / n
    return out


def routing_matrix(qbar, kbar):
    """E[b,h,i,j] = q_bar_i . k_bar_j / sqrt(D)  (float64)."""
    qbar = np.asarray(qbar, dtype=np.float64)
    kbar = np.asarray(kbar, dtype=np.float64)
    D = qbar.shape[-1]
    return np.matmul(qbar, np.swapaxes(kbar, -1, -2)) / np.sqrt(D)


def select_topk(E, R, kmax=None):
    """Keep the R largest scores of every row of E (ties -> lower index).

    Returns (q2k_idx int64 [..., kmax], q2k_num int64 [...], gap float64 [...]):
    kept ids in increasing order followed by -1, the count R, and the score
    gap E_(R) - E_(R+1) between the last kept and the first dropped score
    (+inf when R equals the row length, where nothing competes).
    """
    E = np.asarray(E, dtype=np.float64)
    J = E.shape[-1]
    R = int(R)
    if not 1 <= R <= J:
        raise ValueError("R must lie in [1, J]")
    kmax = R if kmax is None else int(kmax)
    if kmax < R:
        raise ValueError("kmax must be at least R")
    # descending score; a stable sort keeps lower j first among equal scores
    order = np.argsort(-E, axis=-1, kind="stable")
    kept = np.sort(order[..., :R], axis=-1)
    idx = np.full(E.shape[:-1] + (kmax,), -1, dtype=np.int64)
    idx[..., :R] = kept
    num = np.full(E.shape[:-1], R, dtype=np.int64)
    ranked = np.take_along_axis(E, order, axis=-1)
    if R < J:
        gap = ranked[..., R - 1] - ranked[..., R]
    else:
        gap = np.full(E.shape[:-1], np.inf)
    return idx, num, gap
