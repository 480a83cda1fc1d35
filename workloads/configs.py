"""The six workloads, by what they are and their sizes.

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
* h3     -- an H3 reference-to-video sequence in its original order: text (256
            tokens), a reference video (8x48x80), audio (500 tokens), the target
            video (30x48x80); 146676 tokens.  Dense segments in 1D chunks of 64,
            videos in (4,4,4) blocks: 12 prefix blocks + 480 + 1920 video blocks
            (J = 2412); 24 heads, D=128; each video region keeps 10 % of its
            blocks (48 and 192), context rows keep all; bf16 with per-cell
            offsets inside each video region.
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
    "h3": dict(kind="h3", B=1, h=24, segments=[256, (8, 48, 80), 500, (30, 48, 80)], block=(4, 4, 4), D=128,
               keep=0.10, dtype="bf16", seed=6, offset_sigma=1.0),
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
