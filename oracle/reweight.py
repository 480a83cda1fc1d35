"""Spark-Reweight tail summaries and the joint softmax (oracle, float64).

TEST INFRASTRUCTURE ONLY (see the package docstring).

Source: "深度解读|Spark-H3：从注意力几何到稀疏内核代码" (jefxiong.cn):

* section 03: per block B and query q, the exponential mass
  Z_B(q) = sum_{j in B} exp(q.k_j / sqrt(d)) and the unnormalised content
  U_B(q) = sum_{j in B} exp(q.k_j / sqrt(d)) v_j; exact blocks and summarised
  blocks are merged under one shared denominator (one softmax), never as two
  separately normalised outputs;
* section 07: the default representative query of a head is the mean of all
  of that head's (video) queries;
* section 08: with the representative query a, in-block weights
  p_j = softmax_j(a.k_j / sqrt(d)); summary key k~ = sum_j p_j k_j, summary
  value v~ = sum_j p_j v_j; l = log Z_B(a); bias b = l - a.k~ / sqrt(d); a query
  q sees the block through one virtual token with logit q.k~ / sqrt(d) + b and
  value v~.  At q = a the virtual token reproduces Z_B and U_B exactly.
* section 08/09: b equals the entropy of p (between 0 and log m), and the
  virtual logit is the tangent of log Z_B at a, so it never exceeds log Z_B(q).

In the VSA setting a "block" is a tile of the 3D tiling (its true length n_j
tokens, listed in perm), the exact set of a query block is its kept list
(q2k_idx / q2k_num) and every other block of the same (batch, head) enters
through its summary.
"""

import numpy as np


def anchor_queries(Q):
    """Representative query per (batch, head): the mean of all N query rows.

    Q: [B, N, h, D] (any float dtype).  Returns float64 [B, h, D].
    """
    return Q.astype(np.float64).mean(axis=1)


def block_summaries(K, V, perm, block_len, M, anchor, scale=None):
    """Summary key, value, bias and log-mass of every block (section 08).

    K, V: [B, N, h, D]; anchor: [B, h, D]; perm/block_len: the tiling tables
    (block j holds the n_j tokens perm[j*M : j*M + n_j]).

    Returns float64 k_sum [B, h, J, D], v_sum [B, h, J, D], bias [B, h, J]
    and lmass [B, h, J] (= log Z_B(a)).
    """
    B, N, h, D = K.shape
    J = len(block_len)
    scale = 1.0 / np.sqrt(D) if scale is None else float(scale)
    k_sum = np.zeros((B, h, J, D))
    v_sum = np.zeros((B, h, J, D))
    bias = np.zeros((B, h, J))
    lmass = np.zeros((B, h, J))
    a = np.asarray(anchor, dtype=np.float64)
    for j in range(J):
        toks = np.asarray(perm[j * M: j * M + int(block_len[j])])
        k = K[:, toks].astype(np.float64)  # [B, n, h, D]
        v = V[:, toks].astype(np.float64)
        logits = np.einsum("bnhd,bhd->bhn", k, a) * scale
        peak = logits.max(axis=-1, keepdims=True)
        w = np.exp(logits - peak)
        z = w.sum(axis=-1, keepdims=True)
        p = w / z
        k_sum[:, :, j] = np.einsum("bhn,bnhd->bhd", p, k)
        v_sum[:, :, j] = np.einsum("bhn,bnhd->bhd", p, v)
        lmass[:, :, j] = (peak + np.log(z))[..., 0]
        bias[:, :, j] = lmass[:, :, j] - np.einsum("bhd,bhd->bh", a, k_sum[:, :, j]) * scale
    return k_sum, v_sum, bias, lmass


def virtual_logit(q, k_sum, bias, scale):
    """Logit of a block's virtual token for query rows q (section 08)."""
    return (np.asarray(q, dtype=np.float64) @ np.asarray(k_sum, dtype=np.float64)) * scale + bias


def reweight_attention(Q, K, V, perm, block_len, M, q2k_idx, q2k_num, k_sum, v_sum, bias, scale=None,
                       items=None):
    """Exact tokens of the kept blocks plus one virtual token per other block,
    all under one softmax (sections 03 and 08).

    Q, K, V: [B, N, h, D] in the original token order; k_sum/v_sum [B, h, J, D]
    and bias [B, h, J] are the block summaries (any float dtype, upcast
    exactly).  Entry p of row (b, h, i) is kept iff p < q2k_num and
    q2k_idx >= 0; as in the exact path, the tokens of a kept entry count once
    per listing.  Every block that no kept entry names adds its virtual token.
    ``items`` optionally restricts the work to (b, h, i) query blocks; other
    outputs are NaN.

    Returns O float64 [B, N, h, D] and LSE [B, h, N] (natural log).
    """
    B, N, h, D = Q.shape
    J = len(block_len)
    scale = 1.0 / np.sqrt(D) if scale is None else float(scale)
    O = np.full((B, N, h, D), np.nan)
    LSE = np.full((B, h, N), np.nan)
    if items is None:
        items = [(b, hh, i) for b in range(B) for hh in range(h) for i in range(J)]
    for (b, hh, i) in items:
        queries = np.asarray(perm[i * M: i * M + int(block_len[i])])
        kept = []
        for p in range(int(q2k_num[b, hh, i])):
            j = int(q2k_idx[b, hh, i, p])
            if j < 0:
                continue
            if j >= J:
                raise IndexError("block index out of range")
            kept.append(j)
        q = Q[b, queries, hh, :].astype(np.float64)
        parts_s, parts_v = [], []
        if kept:
            toks = np.concatenate([np.asarray(perm[j * M: j * M + int(block_len[j])]) for j in kept])
            parts_s.append((q @ K[b, toks, hh, :].astype(np.float64).T) * scale)
            parts_v.append(V[b, toks, hh, :].astype(np.float64))
        rest = [j for j in range(J) if j not in kept]
        if rest:
            ks = np.asarray(k_sum[b, hh, rest], dtype=np.float64)
            parts_s.append(virtual_logit(q, ks.T, np.asarray(bias[b, hh, rest], dtype=np.float64), scale))
            parts_v.append(np.asarray(v_sum[b, hh, rest], dtype=np.float64))
        s = np.concatenate(parts_s, axis=1)
        vals = np.concatenate(parts_v, axis=0)
        m = s.max(axis=1, keepdims=True)
        w = np.exp(s - m)
        z = w.sum(axis=1, keepdims=True)
        O[b, queries, hh, :] = (w / z) @ vals
        LSE[b, hh, queries] = (m + np.log(z))[:, 0]
    return O, LSE
