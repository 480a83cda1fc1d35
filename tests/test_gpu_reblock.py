"""GPU parity of Spark-Reblock against the float64 oracle: the query-side
second moment, its factor and the unit key features (fp32 bounds), every split
decision of the equal-capacity tree checked node by node on the device's own
node contents (near-ties exempt), the per-head tables, and attention over the
reblocked layouts: every block kept = dense attention (permutation
invariance), routed = the oracle's attention over the device's tables."""

import numpy as np
import pytest
import torch

import oracle
from gpu_util import assert_attn_close, check_topk, to64
from oracle import reblock as rb
from workloads import scaled, vsa_inputs, workload

pytestmark = pytest.mark.gpu

bsa = pytest.importorskip("block_sparse_attention_02_amd")
DEV = torch.device("cuda:0")

# The oracle's unit features are exact (float64); the device computes them in
# fp32 and stores them in fp16, and its splits read the stored values.  Bounds:
# * one component: fp16 rounds a value of magnitude below 1 to within half an
#   ulp, at most 2^-11 of the value (2^-12 in absolute terms for |u_d| < 1);
#   the fp32 pipeline adds far less than 2^-18 (its factor agrees with the
#   oracle's to ~5e-7 relative) -> FEATURE_TOL = 2^-12 + 2^-18;
# * one projection u . v onto a unit direction: |u~ - u| <= 2^-11 |u| = 2^-11
#   for a unit feature, so each token's projection moves by at most 2^-11 and
#   two consecutive tokens of a correctly sorted node can appear inverted by
#   at most 2 * 2^-11 = 2^-10, plus the fp32 dot product's rounding (128 terms
#   of magnitude <= 1: below 2^-16) -> SPLIT_EPS = 2^-10 + 2^-16;
# * the direction: the fp16 features perturb the centred landmarks' Gram by at
#   most 2 * 2^-11 of its norm, which bounds the Rayleigh-quotient shortfall of
#   the device's principal axis against the oracle's on the exact landmarks ->
#   SPLIT_TAU = 2 * 2^-11 (rounded up to 1e-3).  32 nearly isotropic landmarks
#   have close leading eigenvalues, so the two sides may end on different,
#   equally principal axes: the direction is checked for validity rather than
#   equality (the oracle's check_splits).
FEATURE_TOL = 2.0 ** -12 + 2.0 ** -18
SPLIT_EPS = 2.0 ** -10 + 2.0 ** -16
SPLIT_TAU = 1e-3

CFGS = {
    "video_2k_d128": (scaled("video", grid=(8, 16, 16), h=2), 64),
    "ragged_d64": (scaled("video", grid=(7, 9, 13), h=2, D=64), 64),      # 819 tokens: a 51-token last leaf
    "m32": (scaled("video", grid=(6, 12, 20), h=2), 32),
    "root_7400_d64": (scaled("video", grid=(8, 25, 37), h=1, D=64), 64),  # a root above 4096 tokens: the 8192-capacity level
    "m16_d64": (scaled("video", grid=(5, 8, 13), h=2, D=64), 16),         # 520 tokens in 33 leaves of 16 (the last short)
}


def _check_head(x, geom_M, hh, levels, dirs, features, moment, factor, what):
    Q = to64(x["q"][:, :, hh:hh + 1])
    K = to64(x["k"][:, :, hh:hh + 1])
    Mq = rb.second_moment(Q)[0, 0]
    dm = float(np.max(np.abs(to64(moment[hh]) - Mq)) / np.abs(Mq).max())
    Lq = rb.metric_factor(Mq)
    dl = float(np.max(np.abs(to64(factor[hh]) - Lq)) / np.abs(Lq).max())
    U = rb.key_features(K, Q)[0, 0]
    du = float(np.max(np.abs(to64(features[hh]) - U)))
    orders = [lv[hh].cpu().numpy().astype(np.int64) for lv in levels]
    dh = [to64(d[hh]) for d in dirs]
    splits, viol, inv, short = rb.check_splits(U, orders, dh, geom_M, SPLIT_EPS, SPLIT_TAU)
    print("%s head %d: moment rel %.3g, factor rel %.3g, features %.3g; %d splits, %d violations, worst inversion "
          "%.3g, worst quotient shortfall %.3g" % (what, hh, dm, dl, du, splits, viol, inv, short), flush=True)
    # fp32 sums of up to 2048 products per chunk (relative error well below 1e-4)
    assert dm <= 1e-4, what + ": moment"
    assert dl <= 1e-3, what + ": factor"
    assert du <= FEATURE_TOL, "%s: features differ by %.3g" % (what, du)
    assert viol == 0
    return orders[-1]


@pytest.mark.parametrize("name", list(CFGS))
def test_reblock_matches_oracle(name):
    cfg, M = CFGS[name]
    x = vsa_inputs(cfg, device=DEV)
    B, N, H, D = x["q"].shape
    perm, block_len, moment, factor, features, levels, dirs = bsa.spark_reblock(x["q"], x["k"], M=M, debug=True)
    torch.cuda.synchronize()
    J = block_len.numel()
    for hh in range(H):
        final = _check_head(x, M, hh, levels, dirs, features, moment, factor, name)
        ref_perm, ref_len = rb.reblock_tables(final, M)
        assert np.array_equal(perm[hh].cpu().numpy(), ref_perm)
        assert np.array_equal(block_len.cpu().numpy(), ref_len)
    assert J == -(-N // M)


@pytest.mark.parametrize("name", ["video_2k_d128", "ragged_d64"])
def test_all_blocks_kept_is_dense(name):
    """Permutation invariance: reblocked layout, every block kept, outputs at
    their positions = dense attention (float64 SDPA)."""
    cfg, M = CFGS[name]
    x = vsa_inputs(cfg, device=DEV)
    B, N, H, D = x["q"].shape
    J = -(-N // M)
    out, perm, idx, num = bsa.reblock_forward(x["q"], x["k"], x["v"], J, M=M)
    torch.cuda.synchronize()
    Q, K, V = to64(x["q"]), to64(x["k"]), to64(x["v"])
    for hh in range(H):
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(Q[0, :, hh])[None, None], torch.from_numpy(K[0, :, hh])[None, None],
            torch.from_numpy(V[0, :, hh])[None, None])[0, 0].numpy()
        assert_attn_close(out[0, :, hh], ref, "%s all kept, head %d" % (name, hh))


@pytest.mark.parametrize("name", list(CFGS))
def test_routed_attention_over_reblocked_layout(name):
    """Pool -> route -> TopK -> attention over the per-head layouts: the
    oracle pools, routes and attends with each head's device table; index
    tables bit-exact outside near-ties, outputs within the bf16 tolerance."""
    cfg, M = CFGS[name]
    x = vsa_inputs(cfg, device=DEV)
    B, N, H, D = x["q"].shape
    J = -(-N // M)
    R = max(1, J // 4)
    out, perm, idx, num, lse = bsa.reblock_forward(x["q"], x["k"], x["v"], R, M=M, need_lse=True)
    torch.cuda.synchronize()
    Q, K, V = to64(x["q"]), to64(x["k"]), to64(x["v"])
    block_len = rb.reblock_tables(np.arange(N), M)[1]
    for hh in range(H):
        p = perm[hh].cpu().numpy().astype(np.int64)
        sl = (slice(None), slice(None), slice(hh, hh + 1))
        qbar = oracle.pool_blocks(Q[sl], p, block_len, M)
        kbar = oracle.pool_blocks(K[sl], p, block_len, M)
        E = oracle.routing_matrix(qbar, kbar)
        ref_idx, _, gap = oracle.select_topk(E, R)
        got_idx = idx[:, hh:hh + 1].cpu().numpy()
        check_topk(got_idx, E, R, ref_idx, gap, what="%s head %d" % (name, hh))
        O, LSE = oracle.vsa_attention(Q[sl], K[sl], V[sl], p, block_len, M, got_idx, num[:, hh:hh + 1].cpu().numpy())
        assert_attn_close(out[:, :, hh:hh + 1], O, "%s routed, head %d" % (name, hh))
        assert np.abs(to64(lse[:, hh:hh + 1]) - LSE).max() <= 1e-3


def test_reblock_video_full_size():
    """The video workload at full size (115200 tokens, 24 heads, M = 64): the
    tree of heads 0 and 13 checked split by split, every head's table a
    permutation with full leaves."""
    cfg = workload("video")
    x = vsa_inputs(cfg, device=DEV)
    B, N, H, D = x["q"].shape
    print("reblock video full size", flush=True)
    perm, block_len, moment, factor, features, levels, dirs = bsa.spark_reblock(x["q"], x["k"], M=64, debug=True)
    torch.cuda.synchronize()
    assert levels.shape[0] == 12 and block_len.numel() == 1800 and bool((block_len == 64).all())
    srt = torch.sort(perm.long(), dim=1).values
    assert torch.equal(srt, torch.arange(N, device=DEV).expand(H, N))
    for hh in (0, 13):
        _check_head(x, 64, hh, levels, dirs, features, moment, factor, "video full size")


def test_reblock_is_deterministic():
    """Two runs on the same inputs give the same tables bit for bit (no
    floating-point atomics: fixed reduction orders, stable sorts)."""
    cfg, M = CFGS["root_7400_d64"]
    x = vsa_inputs(cfg, device=DEV)
    p1, l1 = bsa.spark_reblock(x["q"], x["k"], M=M)
    p2, l2 = bsa.spark_reblock(x["q"], x["k"], M=M)
    torch.cuda.synchronize()
    assert torch.equal(p1, p2) and torch.equal(l1, l2)


def test_two_batch_entries_equal_single_batch_runs():
    """Batch strides and the per-(batch, head) tables: with two batch entries
    the layout of entry b and the routed attention over it are bitwise those
    of a run on entry b alone (which the tests above check against the
    oracle)."""
    cfg, M = scaled("video", B=2, grid=(8, 16, 16), h=2), 64
    x = vsa_inputs(cfg, device=DEV)
    B, N, H, D = x["q"].shape
    J = -(-N // M)
    R = max(1, J // 4)
    perm2, len2 = bsa.spark_reblock(x["q"], x["k"], M=M)
    out2, _, idx2, num2 = bsa.reblock_forward(x["q"], x["k"], x["v"], R, M=M)
    torch.cuda.synchronize()
    for b in range(B):
        xb = {n: t[b:b + 1] for n, t in x.items()}
        perm1, len1 = bsa.spark_reblock(xb["q"], xb["k"], M=M)
        out1, _, idx1, num1 = bsa.reblock_forward(xb["q"], xb["k"], xb["v"], R, M=M)
        torch.cuda.synchronize()
        assert torch.equal(perm2[b * H:(b + 1) * H], perm1), "batch %d: layout differs" % b
        assert torch.equal(len2, len1)
        assert torch.equal(idx2[b], idx1[0]) and torch.equal(num2[b], num1[0]), "batch %d: index table" % b
        assert torch.equal(out2[b].view(torch.int16), out1[0].view(torch.int16)), "batch %d: output" % b
