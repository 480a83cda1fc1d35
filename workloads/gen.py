"""Seeded generators for the five workloads (data only).

Draw order, per workload (one ``torch.Generator`` seeded with ``seed``):

vsa   Z_q, Z_k, Z_v ~ N(0,1) [B, N, h, D] float32 in token order
      (token id = t*H*W + y*W + x, i.e. the C-order flattening of the grid);
      then, when offset_sigma > 0, one offset field per tensor (q, k, v order)
      ~ N(0, sigma^2) of shape [B, h, ceil(T/cT), ceil(H/cH), ceil(W/cW), D],
      constant over each (cT, cH, cW) cell of the grid and added to every
      token of the cell; finally cast to the workload dtype (bf16: RNE).
h3    Z_q, Z_k, Z_v ~ N(0,1) [B, N, h, D] float32 over the whole sequence in
      original order; then, when offset_sigma > 0, for each video region in
      order and each of q, k, v, an offset field ~ N(0, sigma^2) of shape
      [B, h, ceil(T/cT), ceil(H/cH), ceil(W/cW), D] added to the region's
      tokens (dense segments get none); cast to the workload dtype.
nsa   q [B,T,HQ,D], k [B,T,H,D], v [B,T,H,D] ~ N(0,1) -> bf16; block counts
      U{1..S} [B,T,H]; per chunk of tokens, uniform priorities [B,n,H,NB].
      A token's row holds its own block t // BS plus the c-1 lowest-priority
      blocks strictly before it, c = min(count, t // BS + 1); ascending,
      -1 padded to S.  The returned counts are c.
msa   q [B,N,Hq,D], k, v [B,N,Hkv,D] ~ N(0,1) -> bf16; per KV head a random
      popularity rank of the NB blocks (randperm), weight (rank+1)^-zipf;
      per chunk of positions, Gumbel noise [B,n,Hkv,NB].  A row holds block 0
      and the position's own block, then the highest log-weight + Gumbel
      scores among the other visible blocks (weighted sampling without
      replacement), min(k, own block + 1) entries, ascending, -1 padded to k.
"""

import math

import numpy as np
import torch

_DT = {"bf16": torch.bfloat16, "f32": torch.float32}
_CHUNK = 4096


def _gen(device, seed):
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def vsa_inputs(cfg, device="cpu"):
    """Q, K, V [B, N, h, D] for a VSA workload (dict of tensors)."""
    T, H, W = cfg["grid"]
    B, h, D = cfg["B"], cfg["h"], cfg["D"]
    N = T * H * W
    g = _gen(device, cfg["seed"])
    out = {}
    for name in ("q", "k", "v"):
        out[name] = torch.randn((B, N, h, D), generator=g, device=device,
                                dtype=torch.float32)
    sigma = float(cfg.get("offset_sigma", 0.0))
    if sigma > 0.0:
        cT, cH, cW = cfg.get("offset_cell", cfg["block"])
        nT, nH, nW = -(-T // cT), -(-H // cH), -(-W // cW)
        for name in ("q", "k", "v"):
            c = torch.randn((B, h, nT, nH, nW, D), generator=g, device=device,
                            dtype=torch.float32) * sigma
            field = (c.repeat_interleave(cT, 2).repeat_interleave(cH, 3)
                     .repeat_interleave(cW, 4)[:, :, :T, :H, :W])
            field = field.permute(0, 2, 3, 4, 1, 5).reshape(B, N, h, D)
            out[name] += field
            del c, field
    dt = _DT[cfg["dtype"]]
    return {k_: v_.to(dt) for k_, v_ in out.items()}


def h3_inputs(cfg, device="cpu"):
    """Q, K, V [B, N, h, D] of a multi-region sequence (dict of tensors)."""
    B, h, D = cfg["B"], cfg["h"], cfg["D"]
    segs = cfg["segments"]
    sizes = [s if isinstance(s, int) else s[0] * s[1] * s[2] for s in segs]
    N = sum(sizes)
    g = _gen(device, cfg["seed"])
    out = {name: torch.randn((B, N, h, D), generator=g, device=device, dtype=torch.float32)
           for name in ("q", "k", "v")}
    sigma = float(cfg.get("offset_sigma", 0.0))
    if sigma > 0.0:
        cT, cH, cW = cfg.get("offset_cell", cfg["block"])
        off = 0
        for s, n in zip(segs, sizes):
            if not isinstance(s, int):
                T, H, W = s
                nT, nH, nW = -(-T // cT), -(-H // cH), -(-W // cW)
                for name in ("q", "k", "v"):
                    c = torch.randn((B, h, nT, nH, nW, D), generator=g, device=device, dtype=torch.float32) * sigma
                    field = (c.repeat_interleave(cT, 2).repeat_interleave(cH, 3)
                             .repeat_interleave(cW, 4)[:, :, :T, :H, :W])
                    out[name][:, off:off + n] += field.permute(0, 2, 3, 4, 1, 5).reshape(B, n, h, D)
                    del c, field
            off += n
    dt = _DT[cfg["dtype"]]
    return {k_: v_.to(dt) for k_, v_ in out.items()}


def kept_lists(B, h, J, kmax, seed, device="cpu"):
    """Seeded kept lists for block-selected attention: q2k_idx int32
    [B, h, J, kmax] (ascending, -1 fill) and q2k_num int32 [B, h, J].  Row
    counts are uniform in [0, kmax]; row 0 of every (b, h) keeps nothing and
    row 1 keeps min(kmax, J) blocks, so both extremes always occur."""
    g = np.random.default_rng(seed)
    idx = np.full((B, h, J, kmax), -1, dtype=np.int32)
    num = np.zeros((B, h, J), dtype=np.int32)
    for b in range(B):
        for hh in range(h):
            for i in range(J):
                n = int(g.integers(0, min(kmax, J) + 1))
                if i == 0:
                    n = 0
                elif i == 1:
                    n = min(kmax, J)
                idx[b, hh, i, :n] = np.sort(g.choice(J, size=n, replace=False))
                num[b, hh, i] = n
    return torch.from_numpy(idx).to(device), torch.from_numpy(num).to(device)


def coarse_gate(h, D, seed, device="cpu"):
    """Gate of the coarse pooled-V branch, float32 [h, D]: N(0, 0.5^2) per
    head and channel (a stand-in for a trained gate; zero means no branch)."""
    g = _gen(device, seed)
    return torch.randn((h, D), generator=g, device=device, dtype=torch.float32) * 0.5


def _sorted_padded(sel, limit):
    """Sort a row ascending and turn entries >= limit into -1 (at the end)."""
    sel = torch.sort(sel, dim=-1).values
    return torch.where(sel >= limit, torch.full_like(sel, -1), sel)


def nsa_inputs(cfg, device="cpu"):
    """q, k, v, block_indices [B,T,H,S] int32, block_counts [B,T,H] int32."""
    B, T, HQ, H, D = cfg["B"], cfg["T"], cfg["HQ"], cfg["H"], cfg["D"]
    BS, S = cfg["BS"], cfg["S"]
    g = _gen(device, cfg["seed"])
    dt = _DT[cfg["dtype"]]
    q = torch.randn((B, T, HQ, D), generator=g, device=device).to(dt)
    k = torch.randn((B, T, H, D), generator=g, device=device).to(dt)
    v = torch.randn((B, T, H, D), generator=g, device=device).to(dt)
    counts = torch.randint(1, S + 1, (B, T, H), generator=g, device=device)
    NB = -(-T // BS)
    blk = torch.arange(NB, device=device)
    idx = torch.empty((B, T, H, S), dtype=torch.int64, device=device)
    cnt = torch.empty((B, T, H), dtype=torch.int64, device=device)
    for t0 in range(0, T, _CHUNK):
        t1 = min(T, t0 + _CHUNK)
        cur = torch.arange(t0, t1, device=device) // BS                # [n]
        c = torch.minimum(counts[:, t0:t1], (cur + 1)[None, :, None])  # [B,n,H]
        pri = torch.rand((B, t1 - t0, H, NB), generator=g, device=device)
        earlier = blk[None, None, None, :] < cur[None, :, None, None]
        pri = torch.where(earlier, pri, torch.full_like(pri, 2.0))
        m = min(S - 1, NB)
        others = torch.argsort(pri, dim=-1)[..., :m]
        take = torch.arange(m, device=device) < (c - 1)[..., None]
        others = torch.where(take, others, torch.full_like(others, NB))
        own = cur[None, :, None, None].expand(B, t1 - t0, H, 1)
        sel = torch.cat([own, others], dim=-1)
        if sel.shape[-1] < S:
            pad = torch.full(sel.shape[:-1] + (S - sel.shape[-1],), NB,
                             dtype=sel.dtype, device=device)
            sel = torch.cat([sel, pad], dim=-1)
        idx[:, t0:t1] = _sorted_padded(sel, NB)
        cnt[:, t0:t1] = c
    return q, k, v, idx.to(torch.int32), cnt.to(torch.int32)


def msa_inputs(cfg, device="cpu"):
    """q, k, v and q2k [B, N, Hkv, k] int32 (ascending, -1 padded)."""
    B, N, Hq, Hkv, D = cfg["B"], cfg["N"], cfg["Hq"], cfg["Hkv"], cfg["D"]
    BK, ks, zipf = cfg["BK"], cfg["k"], float(cfg.get("zipf", 1.1))
    g = _gen(device, cfg["seed"])
    dt = _DT[cfg["dtype"]]
    q = torch.randn((B, N, Hq, D), generator=g, device=device).to(dt)
    k = torch.randn((B, N, Hkv, D), generator=g, device=device).to(dt)
    v = torch.randn((B, N, Hkv, D), generator=g, device=device).to(dt)
    NB = -(-N // BK)
    rank = torch.stack([torch.randperm(NB, generator=g, device=device)
                        for _ in range(Hkv)])                          # [Hkv, NB]
    logw = -zipf * torch.log(rank.to(torch.float32) + 1.0)
    blk = torch.arange(NB, device=device)
    out = torch.empty((B, N, Hkv, ks), dtype=torch.int64, device=device)
    m = min(ks, NB)
    for i0 in range(0, N, _CHUNK):
        i1 = min(N, i0 + _CHUNK)
        cur = torch.arange(i0, i1, device=device) // BK                # [n]
        u = torch.rand((B, i1 - i0, Hkv, NB), generator=g, device=device)
        u = u.clamp_(1e-20, 1.0 - 1e-7)
        score = logw[None, None, :, :] - torch.log(-torch.log(u))
        vis = blk[None, None, None, :] <= cur[None, :, None, None]
        must = (blk[None, None, None, :] == 0) | (blk[None, None, None, :] == cur[None, :, None, None])
        score = torch.where(vis, score, torch.full_like(score, -math.inf))
        score = torch.where(must, torch.full_like(score, math.inf), score)
        top = torch.topk(score, m, dim=-1).indices                     # [B,n,Hkv,m]
        kk = torch.minimum(torch.full_like(cur, ks), cur + 1)          # [n]
        keep = torch.arange(m, device=device)[None, None, None, :] < kk[None, :, None, None]
        sel = torch.where(keep, top, torch.full_like(top, NB))
        if m < ks:
            pad = torch.full(sel.shape[:-1] + (ks - m,), NB, dtype=sel.dtype, device=device)
            sel = torch.cat([sel, pad], dim=-1)
        out[:, i0:i1] = _sorted_padded(sel, NB)
    return q, k, v, out.to(torch.int32)
