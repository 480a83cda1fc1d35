"""Work accounting for the throughput figures (host-side bookkeeping).

The pages count attention work as FLOPs = 4 * Hq * N * d * k * B_k ("MSA 为什么
采用 KV-outer Sparse Attention Forward", section 3.1, eq. (13,15)); for VSA the
kept keys per query are R blocks of M tokens ("VSA 实现详解", section 7: the
sparse QK pair count is J * R * M^2).  ``nominal`` figures use those formulas;
``valid`` figures count the query-key pairs that are actually unmasked (edge
blocks shorter than M, causal masks, padded selections).
"""

import torch


def vsa_nominal_flops(B, h, N, D, R, M):
    """4 * B * h * N * D * R * M."""
    return 4.0 * B * h * N * D * R * M


def vsa_valid_pairs(block_len, q2k_idx, q2k_num):
    """Number of unmasked (query, key) pairs of a VSA index table (all heads)."""
    bl = block_len.to(torch.int64)
    kmax = q2k_idx.shape[-1]
    idx = q2k_idx.to(torch.int64)
    slot = torch.arange(kmax, device=idx.device)
    live = (idx >= 0) & (idx < bl.numel()) & (slot < q2k_num.to(torch.int64)[..., None])
    keys = torch.where(live, bl[idx.clamp(min=0, max=bl.numel() - 1)], torch.zeros_like(idx)).sum(-1)   # [B,h,J]
    return int((keys * bl[None, None, :]).sum().item())


def nsa_nominal_flops(block_counts, BS, G, D):
    """4 * G * D * BS * sum(block_counts): every counted block taken as full."""
    return 4.0 * G * D * BS * float(block_counts.to(torch.float64).sum().item())


def kvouter_nominal_flops(q2k, BK, G, D):
    """4 * G * D * BK * (number of valid selections)."""
    return 4.0 * G * D * BK * float((q2k >= 0).sum().item())


def selection_valid_pairs(sel, counts, BS, T, G, causal=True):
    """Unmasked (query, key) pairs of a token-mode selection [B, T, Hkv, S]
    (NSA block_indices, or MSA q2k with counts=None): entries p < count with
    0 <= id and id * BS < T; key positions <= t when causal; G query heads
    per KV head."""
    idx = sel.to(torch.int64)
    S = idx.shape[-1]
    t = torch.arange(T, device=idx.device).view(1, T, 1, 1)
    live = (idx >= 0) & (idx * BS < T)
    if counts is not None:
        live &= torch.arange(S, device=idx.device) < counts.to(torch.int64)[..., None]
    start = idx * BS
    end = torch.clamp(start + BS, max=T)
    if causal:
        end = torch.minimum(end, t + 1)
    keys = torch.where(live, torch.clamp(end - start, min=0), torch.zeros_like(idx))
    return int(keys.sum().item()) * G
