"""Exact sparse attention over selected blocks, and the KV-outer algebra
(oracle, float64).

Sources:
* "VSA 实现详解：三维分块、均值路由与块稀疏 Attention", section 4 (every query of
  block i sees all valid keys of every kept block; weights are per token),
  section 6.3 (per query block: loop over the q2k_num kept blocks, mask keys
  beyond the true length of each, softmax over the union), section 6.5 (a row
  with no visible key gives a zero output) and section 8 (the result equals
  explicit masked attention in the original token order).  No causal mask.
* "NSA 算子解析（Torch/Tilelang）", "Torch朴素实现": per (batch, token, query
  head) the keys are the tokens of the selected blocks of KV head hq // G; a
  key is dropped when its position exceeds the query position or its block
  slot is not below the block count; scale = D ** -0.5.
* "MSA 为什么采用 KV-outer Sparse Attention Forward", section 6.1 (K1: per
  selected block s, L_s = log sum_j exp S_j and O_s = sum_j exp(S_j - L_s) V_j)
  and section 6.2 (K2: a = max L_s, L = a + log sum exp(L_s - a),
  O = sum_s exp(L_s - L) O_s, equal to one global softmax).

All functions compute the plain definitions: gather the allowed keys, form the
logits, one softmax, one weighted sum.  LSE values use the natural logarithm.
"""

import numpy as np


def _softmax_rows(s):
    """Row softmax weights and log-sum-exp of a float64 logit matrix."""
    m = s.max(axis=-1, keepdims=True)
    w = np.exp(s - m)
    z = w.sum(axis=-1, keepdims=True)
    return w / z, (m + np.log(z))[..., 0]


def vsa_attention(Q, K, V, perm, block_len, M, q2k_idx, q2k_num, scale=None,
                  items=None):
    """Block-selected attention (VSA mode).

    Q, K, V: [B, N, h, D] in the original token order (any float dtype; values
    are upcast exactly to float64).  perm/block_len: the tiling tables.
    q2k_idx [B, h, J, kmax], q2k_num [B, h, J]: entry p of row (b, h, i) counts
    iff p < q2k_num and q2k_idx >= 0.  ``items`` optionally restricts the work
    to a list of (b, h, i) query blocks; other outputs are NaN.

    Returns O float64 [B, N, h, D] (original token order) and LSE [B, h, N].
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
        keys = []
        for p in range(int(q2k_num[b, hh, i])):
            j = int(q2k_idx[b, hh, i, p])
            if j < 0:
                continue
            if j >= J:
                raise IndexError("block index out of range")
            keys.append(np.asarray(perm[j * M: j * M + int(block_len[j])]))
        if not keys:
            O[b, queries, hh, :] = 0.0
            LSE[b, hh, queries] = -np.inf
            continue
        keys = np.concatenate(keys)
        q = Q[b, queries, hh, :].astype(np.float64)
        k = K[b, keys, hh, :].astype(np.float64)
        v = V[b, keys, hh, :].astype(np.float64)
        w, lse = _softmax_rows((q @ k.T) * scale)
        O[b, queries, hh, :] = w @ v
        LSE[b, hh, queries] = lse
    return O, LSE


def _selected_keys(blocks, count, BS, T, t, causal):
    """Key positions of the selected blocks of one (token, KV head) row."""
    keys = []
    for p in range(len(blocks)):
        if count is not None and p >= count:
            break
        blk = int(blocks[p])
        if blk < 0:
            continue
        if blk * BS >= T:
            raise IndexError("block index out of range")
        for u in range(BS):
            pos = blk * BS + u
            if pos >= T:
                break
            if causal and pos > t:
                break
            keys.append(pos)
    return np.asarray(keys, dtype=np.int64)


def nsa_attention(q, k, v, block_indices, block_counts, BS, causal=True,
                  scale=None, tokens=None):
    """NSA selected-branch attention with GQA.

    q [B, T, HQ, D], k/v [B, T, H, D], block_indices [B, T, H, S] (-1 padded),
    block_counts [B, T, H] or None (all S entries count).  Query head hq reads
    KV head hq // (HQ // H).  ``tokens`` optionally restricts the work to a
    list of (b, t); other outputs are NaN.  Returns o [B, T, HQ, D], lse
    [B, T, HQ].
    """
    B, T, HQ, D = q.shape
    H = k.shape[2]
    if HQ % H:
        raise ValueError("HQ must be a multiple of H")
    G = HQ // H
    scale = 1.0 / np.sqrt(D) if scale is None else float(scale)
    o = np.full((B, T, HQ, D), np.nan)
    lse = np.full((B, T, HQ), np.nan)
    if tokens is None:
        tokens = [(b, t) for b in range(B) for t in range(T)]
    for (b, t) in tokens:
        for r in range(H):
            cnt = None if block_counts is None else int(block_counts[b, t, r])
            keys = _selected_keys(block_indices[b, t, r], cnt, BS, T, t, causal)
            heads = slice(r * G, (r + 1) * G)
            if keys.size == 0:
                o[b, t, heads, :] = 0.0
                lse[b, t, heads] = -np.inf
                continue
            qq = q[b, t, heads, :].astype(np.float64)          # [G, D]
            kk = k[b, keys, r, :].astype(np.float64)           # [n, D]
            vv = v[b, keys, r, :].astype(np.float64)
            w, l_ = _softmax_rows((qq @ kk.T) * scale)
            o[b, t, heads, :] = w @ vv
            lse[b, t, heads] = l_
    return o, lse


def kvouter_partials(q, k, v, q2k, BK, causal=True, scale=None, q2k_cnt=None,
                     positions=None):
    """K1 intermediates of the KV-outer schedule.

    q [B, N, Hq, D], k/v [B, N, Hkv, D], q2k [B, N, Hkv, ks] (-1 padded),
    optional q2k_cnt [B, N, Hkv].  The valid entries of a row (p < cnt when
    counts are given, id >= 0) are taken in increasing block order; slot s is
    the rank of a block in that order.  For slot s with visible key set J_s:
    L_s = log sum_j exp S_j, O_s = sum_j exp(S_j - L_s) v_j, S_j = q.k_j*scale;
    an empty J_s gives L_s = -inf and O_s = 0.

    Returns O_buf [B, ks, N, Hq, D], LSE_buf [B, ks, N, Hq] (unused slots:
    O = 0, L = -inf) and nslot [B, N, Hkv].  With ``positions`` (a list of
    (b, i)) only those rows are computed and the arrays are compact, indexed by
    the list order: O_buf [P, ks, Hq, D], LSE_buf [P, ks, Hq], nslot [P, Hkv].
    """
    B, N, Hq, D = q.shape
    Hkv = k.shape[2]
    ks = q2k.shape[-1]
    G = Hq // Hkv
    scale = 1.0 / np.sqrt(D) if scale is None else float(scale)
    compact = positions is not None
    if positions is None:
        positions = [(b, i) for b in range(B) for i in range(N)]
    P = len(positions)
    O_buf = np.zeros((P, ks, Hq, D))
    LSE_buf = np.full((P, ks, Hq), -np.inf)
    nslot = np.zeros((P, Hkv), dtype=np.int64)
    for n, (b, i) in enumerate(positions):
        for r in range(Hkv):
            row = q2k[b, i, r]
            cnt = ks if q2k_cnt is None else int(q2k_cnt[b, i, r])
            blocks = sorted(int(x) for x in row[:cnt] if x >= 0)
            nslot[n, r] = len(blocks)
            heads = slice(r * G, (r + 1) * G)
            qq = q[b, i, heads, :].astype(np.float64)
            for s, blk in enumerate(blocks):
                keys = _selected_keys([blk], None, BK, N, i, causal)
                if keys.size == 0:
                    continue
                kk = k[b, keys, r, :].astype(np.float64)
                vv = v[b, keys, r, :].astype(np.float64)
                w, l_ = _softmax_rows((qq @ kk.T) * scale)
                O_buf[n, s, heads, :] = w @ vv
                LSE_buf[n, s, heads] = l_
    if compact:
        return O_buf, LSE_buf, nslot
    # full layout: [B, ks, N, Hq, D], [B, ks, N, Hq], [B, N, Hkv]
    O_full = O_buf.reshape(B, N, ks, Hq, D).transpose(0, 2, 1, 3, 4)
    L_full = LSE_buf.reshape(B, N, ks, Hq).transpose(0, 2, 1, 3)
    return np.ascontiguousarray(O_full), np.ascontiguousarray(L_full), nslot.reshape(B, N, Hkv)


def lse_combine(O_buf, LSE_buf, nslot, G):
    """K2: exact merge of per-slot partials with their log-sum-exps.

    O_buf [B, ks, N, Hq, D], LSE_buf [B, ks, N, Hq], nslot [B, N, Hkv] with
    Hq = G * Hkv; slots s < nslot[b, i, hq // G] are valid.  Returns
    O [B, N, Hq, D] and L [B, N, Hq]; rows with no slot, or whose slots are
    all -inf, give O = 0 and L = -inf.
    """
    O_buf = np.asarray(O_buf, dtype=np.float64)
    LSE_buf = np.asarray(LSE_buf, dtype=np.float64)
    B, ks, N, Hq, D = O_buf.shape
    n = np.asarray(nslot)[:, :, np.arange(Hq) // G]                # [B, N, Hq]
    valid = np.arange(ks)[None, :, None, None] < n[:, None, :, :]  # [B, ks, N, Hq]
    ls = np.where(valid, LSE_buf, -np.inf)
    a = ls.max(axis=1)                                             # [B, N, Hq]
    live = np.isfinite(a)
    a0 = np.where(live, a, 0.0)
    with np.errstate(invalid="ignore", divide="ignore"):
        L = a0 + np.log(np.exp(ls - a0[:, None]).sum(axis=1))
        L = np.where(live, L, -np.inf)
        w = np.where(valid & live[:, None], np.exp(ls - np.where(live, L, 0.0)[:, None]), 0.0)
    parts = np.where(valid[..., None], O_buf, 0.0)
    O = (w[..., None] * parts).sum(axis=1)
    return O, L
