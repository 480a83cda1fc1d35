"""Coarse pooled-V branch (oracle, float64).

TEST INFRASTRUCTURE ONLY (see the package docstring).

Source: "VSA 实现详解：三维分块、均值路由与块稀疏 Attention", section 6.7: coarse
attention over all logical blocks, C = softmax(E) V_bar, with E the routing
matrix of section 2.2 and V_bar the per-block means of V (pooled like Q_bar and
K_bar, section 2.1); each query block's row of C is broadcast to the tokens of
that block and added to the sparse output under a gate g:
O = O_sparse + g * broadcast(C).  With g = 0 the branch changes nothing.

Reading: g is one value per (head, channel), g[h, d]; a scalar gate per head
is the case of equal entries.
"""

import numpy as np


def coarse_attention(E, vbar):
    """C[b, h, i, :] = sum_j softmax_j(E[b, h, i, :]) vbar[b, h, j, :].

    E: [B, h, J, J] routing scores (already scaled); vbar: [B, h, J, D].
    Returns float64 [B, h, J, D].
    """
    E = np.asarray(E, dtype=np.float64)
    m = E.max(axis=-1, keepdims=True)
    w = np.exp(E - m)
    w /= w.sum(axis=-1, keepdims=True)
    return np.einsum("bhij,bhjd->bhid", w, np.asarray(vbar, dtype=np.float64))


def add_coarse(O, C, gate, perm, block_len, M):
    """O + g * broadcast(C): every valid token of block i gets gate[h] * C[b, h, i].

    O: [B, N, h, D] (float64 copy returned), C: [B, h, J, D], gate: [h, D].
    """
    O = np.array(O, dtype=np.float64, copy=True)
    C = np.asarray(C, dtype=np.float64)
    g = np.asarray(gate, dtype=np.float64)
    for i in range(len(block_len)):
        toks = np.asarray(perm[i * M: i * M + int(block_len[i])])
        O[:, toks] += (g[None] * C[:, :, i])[:, None]
    return O
