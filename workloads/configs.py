"""The five workloads, by what they are and their sizes.

* tiny   -- the walkthrough's teaching grid: 4x4x4 tokens in (4,2,2) blocks,
            one head, D=64, keep 2 of 4 blocks, float32 inputs.
* small  -- an 8x16x16 video grid in (4,4,4) blocks (32 blocks of 64), 8 heads,
            D=64, keep 25% (8 blocks), bf16.
* video  -- a 30x48x80 video-DiT grid in (4,4,4) blocks: 1920 blocks, the last
            temporal slab holds 32-token edge blocks; 24 heads, D=128, keep 10%
            (192 blocks); bf16 with a unit-variance offset shared by each
            4x4x4 cell of the grid (spatial locality).
* nsa    -- NSA selected branch: 32768 tokens, 64 query heads over 4 KV heads
            (G=16), D=128, blocks of 64, up to 16 selected blocks, causal.
* msa    -- MSA KV-outer prefill: 65536 tokens, 64 query heads over 4 KV heads,
            D=128, KV blocks of 128, 16 selected blocks per query and KV head,
            causal; selections always hold block 0 and the query's own block,
            the rest follow a Zipf(1.1) popularity per KV head.
"""

import copy

WORKLOADS = {
    "tiny": dict(kind="vsa", B=1, h=1, grid=(4, 4, 4), block=(4, 2, 2), D=64,
                 R=2, dtype="f32", seed=1, offset_sigma=0.0),
    "small": dict(kind="vsa", B=1, h=8, grid=(8, 16, 16), block=(4, 4, 4), D=64,
                  R=8, dtype="bf16", seed=2, offset_sigma=0.0),
    "video": dict(kind="vsa", B=1, h=24, grid=(30, 48, 80), block=(4, 4, 4),
                  D=128, R=192, dtype="bf16", seed=3, offset_sigma=1.0),
    "nsa": dict(kind="nsa", B=1, T=32768, HQ=64, H=4, D=128, BS=64, S=16,
                causal=True, dtype="bf16", seed=4),
    "msa": dict(kind="msa", B=1, N=65536, Hq=64, Hkv=4, D=128, BK=128, k=16,
                causal=True, dtype="bf16", seed=5, zipf=1.1),
}


def workload(name):
    """A fresh copy of a named workload's parameters."""
    return copy.deepcopy(WORKLOADS[name])


def scaled(name, **overrides):
    """A named workload with some parameters replaced (same structure, smaller
    sizes for tests the oracle finishes in seconds)."""
    cfg = workload(name)
    cfg.update(overrides)
    return cfg
