"""GPU parity of the Spark-Reweight path against the float64 oracle: the
anchor and block summaries (bf16 rounding bounds), attention with virtual
tokens (bf16 attention tolerance), exactness at the anchor end to end, and the
video workload at full size on sampled query blocks."""

import math

import numpy as np
import pytest
import torch

import oracle
from gpu_util import assert_attn_close, to64
from workloads import kept_lists, scaled, vsa_inputs

pytestmark = pytest.mark.gpu

bsa = pytest.importorskip("block_sparse_attention_02_amd")
DEV = torch.device("cuda:0")


def _setup(cfg):
    T, H, W = cfg["grid"]
    geom = bsa.VsaGeometry((T, H, W), cfg["block"], device=DEV)
    tab = oracle.tile_index(T, H, W, *cfg["block"])
    x = vsa_inputs(cfg, device=DEV)
    return geom, tab, x


SUM_CFGS = {
    "ragged_d128": scaled("video", grid=(6, 12, 20), h=2, R=4),
    "ragged_d64": scaled("video", grid=(7, 9, 13), h=3, D=64, R=3),
    "ragged_d128_b2": scaled("video", B=2, grid=(6, 12, 20), h=2, R=4),
}


@pytest.mark.parametrize("name", list(SUM_CFGS))
def test_summaries_match_oracle(name):
    cfg = SUM_CFGS[name]
    geom, tab, x = _setup(cfg)
    print("summaries", name, cfg["grid"], "J", geom.J, flush=True)
    k_sum, v_sum, b_sum, anchor = bsa.spark_summaries(x["q"], x["k"], x["v"], geom.perm, geom.block_len, geom.J,
                                                      geom.M, need_anchor=True)
    torch.cuda.synchronize()
    Q, K, V = to64(x["q"]), to64(x["k"]), to64(x["v"])
    a = oracle.anchor_queries(Q)
    # the anchor is an fp32 sum of N bf16 rows
    assert np.max(np.abs(to64(anchor) - a)) < 1e-5
    ks, vs, b, _ = oracle.block_summaries(K, V, tab["perm"], tab["block_len"], tab["M"], a)
    # one bf16 rounding of a value computed in fp32
    for got, ref, what in ((k_sum, ks, "k_sum"), (v_sum, vs, "v_sum")):
        err = np.abs(to64(got) - ref)
        tol = 2.0 ** -8 * np.abs(ref) + 1e-4
        assert np.all(err <= tol), "%s: worst excess %.3g" % (what, float((err - tol).max()))
    # the bias uses the stored (rounded) key: it may differ from the unrounded
    # definition by scale * |a| . |k_sum - rn(k_sum)| <= scale * |a| . |k_sum| 2^-8
    scale = 1.0 / math.sqrt(cfg["D"])
    bound = scale * np.einsum("bhd,bhjd->bhj", np.abs(a), np.abs(ks)) * 2.0 ** -8 + 1e-4
    err = np.abs(to64(b_sum) - b)
    assert np.all(err <= bound), "b_sum: worst excess %.3g" % float((err - bound).max())


ATTN_CFGS = {
    # J = 2*6*7 = 84: two summary tiles, the second ragged (20 of 64)
    "two_tiles": scaled("video", grid=(8, 24, 28), h=2, R=6),
    "ragged_blocks": scaled("video", grid=(6, 22, 30), h=2, R=9),
    "d64": scaled("video", grid=(5, 16, 16), h=2, D=64, R=3),
    "two_tiles_b2": scaled("video", B=2, grid=(8, 24, 28), h=2, R=6),
}


@pytest.mark.parametrize("name", list(ATTN_CFGS))
def test_attention_with_summaries_matches_oracle(name):
    """Same inputs on both sides: seeded kept lists (including rows that keep
    nothing and rows that keep the most), oracle summaries rounded to the
    stored dtypes."""
    cfg = ATTN_CFGS[name]
    geom, tab, x = _setup(cfg)
    J, kmax = geom.J, min(cfg["R"] + 3, geom.J)
    idx, num = kept_lists(cfg["B"], cfg["h"], J, kmax, seed=11, device=DEV)
    print("attention+summaries", name, cfg["grid"], "J", J, flush=True)
    Q, K, V = to64(x["q"]), to64(x["k"]), to64(x["v"])
    ks, vs, b, _ = oracle.block_summaries(K, V, tab["perm"], tab["block_len"], tab["M"], oracle.anchor_queries(Q))
    k_sum = torch.from_numpy(ks).to(DEV, torch.bfloat16).contiguous()
    v_sum = torch.from_numpy(vs).to(DEV, torch.bfloat16).contiguous()
    b_sum = torch.from_numpy(b).to(DEV, torch.float32).contiguous()
    out, lse = bsa.attention_vsa(x["q"], x["k"], x["v"], geom.perm, geom.block_len, J, geom.M, idx, num,
                                 need_lse=True, summaries=(k_sum, v_sum, b_sum))
    torch.cuda.synchronize()
    O, LSE = oracle.reweight_attention(Q, K, V, tab["perm"], tab["block_len"], tab["M"], idx.cpu().numpy(),
                                       num.cpu().numpy(), to64(k_sum), to64(v_sum), to64(b_sum))
    assert_attn_close(out, O, "attention+summaries " + name)
    assert np.max(np.abs(to64(lse) - LSE)) < 1e-3


def test_exact_at_anchor_end_to_end():
    """Every query equal to one anchor row: summaries from the GPU and the
    attention with virtual tokens give dense attention over all tokens."""
    cfg = scaled("video", grid=(8, 24, 28), h=2, R=5)
    geom, tab, x = _setup(cfg)
    B, N, h, D = x["q"].shape
    a = x["q"][:, :1].expand(B, N, h, D).contiguous()  # bf16 rows, all equal
    J = geom.J
    idx, num = kept_lists(B, h, J, min(6, J), seed=12, device=DEV)
    summ = bsa.spark_summaries(a, x["k"], x["v"], geom.perm, geom.block_len, J, geom.M)
    out = bsa.attention_vsa(a, x["k"], x["v"], geom.perm, geom.block_len, J, geom.M, idx, num, summaries=summ)
    torch.cuda.synchronize()
    Q, K, V = to64(a), to64(x["k"]), to64(x["v"])
    every = np.broadcast_to(np.arange(J), (B, h, J, J)).copy()
    dense, _ = oracle.vsa_attention(Q, K, V, tab["perm"], tab["block_len"], tab["M"], every,
                                    np.full((B, h, J), J))
    assert_attn_close(out, dense, "exact at the anchor")


def test_all_blocks_kept_equals_plain_path():
    """Rows that keep every block add no virtual token: the summary path gives
    the plain path's result.  The two run different kernels (their sums are
    ordered differently), so both must match dense attention within the
    attention tolerance and each other within two bf16 rounding steps."""
    cfg = scaled("video", grid=(8, 16, 16), h=2, R=4)
    geom, tab, x = _setup(cfg)
    B, N, h, D = x["q"].shape
    J = geom.J
    idx = torch.arange(J, dtype=torch.int32, device=DEV).expand(B, h, J, J).contiguous()
    num = torch.full((B, h, J), J, dtype=torch.int32, device=DEV)
    summ = bsa.spark_summaries(x["q"], x["k"], x["v"], geom.perm, geom.block_len, J, geom.M)
    o1 = bsa.attention_vsa(x["q"], x["k"], x["v"], geom.perm, geom.block_len, J, geom.M, idx, num, summaries=summ)
    o2 = bsa.attention_vsa(x["q"], x["k"], x["v"], geom.perm, geom.block_len, J, geom.M, idx, num)
    torch.cuda.synchronize()
    Q, K, V = to64(x["q"]), to64(x["k"]), to64(x["v"])
    dense, _ = oracle.vsa_attention(Q, K, V, tab["perm"], tab["block_len"], tab["M"], idx.cpu().numpy(),
                                    num.cpu().numpy())
    assert_attn_close(o1, dense, "summaries, every block kept")
    assert_attn_close(o2, dense, "plain, every block kept")
    a, b = o1.float(), o2.float()
    assert bool(((a - b).abs() <= 2.0 ** -6 * b.abs() + 2.0 ** -20).all())


def test_summary_argument_errors():
    cfg = scaled("video", grid=(4, 8, 8), h=1, R=2)
    geom, tab, x = _setup(cfg)
    J = geom.J
    idx, num = kept_lists(1, 1, J, 2, seed=13, device=DEV)
    k_sum, v_sum, b_sum = bsa.spark_summaries(x["q"], x["k"], x["v"], geom.perm, geom.block_len, J, geom.M)
    with pytest.raises(ValueError):
        bsa.attention_vsa(x["q"], x["k"], x["v"], geom.perm, geom.block_len, J, geom.M, idx, num,
                          summaries=(k_sum.float(), v_sum, b_sum))
    # the library itself refuses summaries for blocks of capacity 32
    geom32 = bsa.VsaGeometry((4, 8, 8), (2, 4, 4), device=DEV)
    idx32, num32 = kept_lists(1, 1, geom32.J, 2, seed=14, device=DEV)
    s32 = bsa.spark_summaries(x["q"], x["k"], x["v"], geom32.perm, geom32.block_len, geom32.J, geom32.M)
    with pytest.raises(Exception, match="capacity 64"):
        bsa.attention_vsa(x["q"], x["k"], x["v"], geom32.perm, geom32.block_len, geom32.J, geom32.M, idx32, num32,
                          summaries=s32)


def test_video_full_size_sampled():
    """The video workload at full size (115200 tokens, 24 heads, J = 1920, R = 192
    kept per row from the seeded generator), summaries and attention on the GPU
    as bench.py runs them; the oracle recomputes summaries and sampled query
    blocks of three heads from the same inputs."""
    cfg = scaled("video")
    geom, tab, x = _setup(cfg)
    B, N, h, D = x["q"].shape
    J, R = geom.J, cfg["R"]
    idx, num = kept_lists(B, h, J, R, seed=15, device=DEV)
    print("video full size with summaries, J", J, flush=True)
    summ = bsa.spark_summaries(x["q"], x["k"], x["v"], geom.perm, geom.block_len, J, geom.M)
    out, lse = bsa.attention_vsa(x["q"], x["k"], x["v"], geom.perm, geom.block_len, J, geom.M, idx, num,
                                 need_lse=True, summaries=summ)
    torch.cuda.synchronize()
    heads = [0, 11, 23]
    Q, K, V = (to64(t[:, :, heads]) for t in (x["q"], x["k"], x["v"]))
    ks, vs, b, _ = oracle.block_summaries(K, V, tab["perm"], tab["block_len"], tab["M"], oracle.anchor_queries(Q))
    rng = np.random.default_rng(16)
    blocks = [0, 1, J - 1] + [int(v) for v in rng.choice(J, 5, replace=False)]
    items = [(0, hi, i) for hi in range(len(heads)) for i in blocks]
    hsel = torch.tensor(heads, device=DEV)
    O, LSE = oracle.reweight_attention(Q, K, V, tab["perm"], tab["block_len"], tab["M"],
                                       idx[:, hsel].cpu().numpy(), num[:, hsel].cpu().numpy(), ks, vs, b,
                                       items=items)
    got = to64(out[:, :, heads])
    mask = ~np.isnan(O)
    assert_attn_close(got[mask], O[mask], "video full size, sampled blocks with summaries")
    lmask = ~np.isnan(LSE)
    assert np.max(np.abs(to64(lse[:, heads])[lmask] - LSE[lmask])) < 1e-3
