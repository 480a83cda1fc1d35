"""GPU parity of the coarse pooled-V branch against the float64 oracle: the
branch itself (C = softmax(E) V_bar, fp32 bounds), C from the device's own
routing scores, attention with the gated branch merged into its epilogue
(bf16 attention tolerance) for every kernel family (M = 64, M <= 32, fp32),
a zero gate (bitwise the plain path), the branch together with Spark-Reweight
summaries, argument errors, and the video workload at full size on sampled
query blocks."""

import numpy as np
import pytest
import torch

import oracle
from gpu_util import assert_attn_close, to64
from workloads import coarse_gate, kept_lists, scaled, vsa_inputs, workload

pytestmark = pytest.mark.gpu

bsa = pytest.importorskip("block_sparse_attention_02_amd")
DEV = torch.device("cuda:0")
EPS32 = 2.0 ** -24


def _setup(cfg):
    T, H, W = cfg["grid"]
    geom = bsa.VsaGeometry((T, H, W), cfg["block"], device=DEV)
    tab = oracle.tile_index(T, H, W, *cfg["block"])
    x = vsa_inputs(cfg, device=DEV)
    return geom, tab, x


def _oracle_scores(Q, K, tab):
    qbar = oracle.pool_blocks(Q, tab["perm"], tab["block_len"], tab["M"])
    kbar = oracle.pool_blocks(K, tab["perm"], tab["block_len"], tab["M"])
    return oracle.routing_matrix(qbar, kbar)


def _c_bound(E, vbar, V, J):
    """Error bound of C: the block means (<= 64 rounded fp32 adds of values
    below max|V|), the weights (argument E - m and exp2 rounding, about
    2|E - m| + 2 ulp relative), the J-term fp32 weighted sum, and the products:
    weights and block means each split into bf16 hi + lo and multiplied as
    hi*hi + hi*lo + lo*hi, which drops lo*lo and the two lo roundings (each at
    most 2^-18 of the product, so 3 * 2^-18 relative); a factor 4 of margin."""
    spread = float((E.max(axis=-1) - E.min(axis=-1)).max())
    vmax = float(np.abs(vbar).max())
    fp32 = EPS32 * ((J + 2 * spread + 4) * vmax + 64 * float(np.abs(V).max()))
    return 4 * (fp32 + 3 * 2.0 ** -18 * vmax) + 1e-7


COARSE_CFGS = {
    "tiny_f32": workload("tiny"),                                   # J = 4 (< one row tile), M = 16
    "small": workload("small"),                                     # J = 32, D = 64
    "two_col_steps": scaled("video", grid=(8, 24, 28), h=2, R=6),   # J = 84: 64 + a ragged 20
    "ragged_blocks": scaled("video", grid=(6, 22, 30), h=2, R=9),   # partial blocks on every axis
    "d64_odd": scaled("video", grid=(9, 12, 20), h=3, D=64, R=5),
    "odd_two_chunks": scaled("video", grid=(12, 20, 28), h=2, R=7),  # J = 105: unaligned rows, 64 + 41 columns
    "two_batches": scaled("video", B=2, grid=(8, 24, 28), h=2, R=6),
}


@pytest.mark.parametrize("name", list(COARSE_CFGS))
def test_coarse_matches_oracle(name):
    """Same fp32 scores on both sides (the oracle's, rounded to fp32)."""
    cfg = COARSE_CFGS[name]
    geom, tab, x = _setup(cfg)
    J = geom.J
    print("coarse", name, cfg["grid"], "J", J, flush=True)
    Q, K, V = to64(x["q"]), to64(x["k"]), to64(x["v"])
    E32 = _oracle_scores(Q, K, tab).astype(np.float32)
    E = torch.from_numpy(E32).to(DEV).contiguous()
    C, vbar = bsa.coarse_attention(x["v"], geom.perm, geom.block_len, J, geom.M, E, need_vbar=True)
    torch.cuda.synchronize()
    rv = oracle.pool_blocks(V, tab["perm"], tab["block_len"], tab["M"])
    assert np.max(np.abs(to64(vbar) - rv)) <= 64 * EPS32 * float(np.abs(V).max()) + 1e-7
    rC = oracle.coarse_attention(E32.astype(np.float64), rv)
    err = float(np.max(np.abs(to64(C) - rC)))
    bound = _c_bound(E32, rv, V, J)
    print("%s: C max abs err %.3g (bound %.3g)" % (name, err, bound), flush=True)
    assert err <= bound


def test_coarse_from_routing_scores():
    """C from the device's own scores E (routing output) against the oracle's
    scores from Q and K: the fp32 bound plus the effect of the score error
    (each weight moves by at most 2 max|dE| relative, so C by 2 max|dE| max|V_bar|)."""
    cfg = scaled("video", grid=(12, 16, 20), h=3, R=6)
    geom, tab, x = _setup(cfg)
    B, N, H, D = x["q"].shape
    J = geom.J
    E = torch.empty((B, H, J, J), dtype=torch.float32, device=DEV)
    bsa.pool_route_topk(x["q"], x["k"], geom.perm, geom.block_len, J, geom.M, cfg["R"], scores=E)
    C = bsa.coarse_attention(x["v"], geom.perm, geom.block_len, J, geom.M, E)
    torch.cuda.synchronize()
    Q, K, V = to64(x["q"]), to64(x["k"]), to64(x["v"])
    rE = _oracle_scores(Q, K, tab)
    dE = 2e-5 * max(1.0, float(np.abs(rE).max()))  # the routing step's score tolerance
    assert float(np.max(np.abs(to64(E) - rE))) <= dE
    rv = oracle.pool_blocks(V, tab["perm"], tab["block_len"], tab["M"])
    rC = oracle.coarse_attention(rE, rv)
    err = float(np.max(np.abs(to64(C) - rC)))
    bound = _c_bound(rE, rv, V, J) + 2 * dE * float(np.abs(rv).max())
    print("C from routing scores: max abs err %.3g (bound %.3g)" % (err, bound), flush=True)
    assert err <= bound


ATTN_CFGS = {
    "tiny_f32": workload("tiny"),                                            # fp32 kernel, M = 16
    "small_d64": workload("small"),                                          # M = 64, D = 64
    "video_ragged": scaled("video", grid=(6, 22, 30), h=2, R=9),            # M = 64, D = 128
    "video_m32": scaled("video", grid=(8, 12, 16), h=2, block=(2, 4, 4), R=10),  # M = 32 kernel
    "video_ragged_b2": scaled("video", B=2, grid=(6, 22, 30), h=2, R=9),   # two batch entries
}


@pytest.mark.parametrize("name", list(ATTN_CFGS))
def test_attention_with_coarse_matches_oracle(name):
    """The routed forward with the gated branch: the oracle attends over the
    device's index table (validated on its own by the routing tests) and adds
    the branch computed from its own scores and block means."""
    cfg = ATTN_CFGS[name]
    geom, tab, x = _setup(cfg)
    H, D = cfg["h"], cfg["D"]
    gate = coarse_gate(H, D, seed=31, device=DEV)
    print("attention+coarse", name, cfg["grid"], "J", geom.J, flush=True)
    out, idx, num = bsa.vsa_forward(x["q"], x["k"], x["v"], geom, cfg["R"], gate=gate)
    torch.cuda.synchronize()
    Q, K, V = to64(x["q"]), to64(x["k"]), to64(x["v"])
    O, _ = oracle.vsa_attention(Q, K, V, tab["perm"], tab["block_len"], tab["M"], idx.cpu().numpy(),
                                num.cpu().numpy())
    rv = oracle.pool_blocks(V, tab["perm"], tab["block_len"], tab["M"])
    rC = oracle.coarse_attention(_oracle_scores(Q, K, tab), rv)
    ref = oracle.add_coarse(O, rC, to64(gate), tab["perm"], tab["block_len"], tab["M"])
    assert_attn_close(out, ref, "attention+coarse " + name)
    # the branch is really there: it moves the output by far more than the tolerance
    assert float(np.max(np.abs(ref - O))) > 2e-2


@pytest.mark.parametrize("name", ["tiny_f32", "small_d64", "video_m32"])
def test_zero_gate_is_plain_attention(name):
    """A zero gate (the initial value of a model without a trained gate) adds
    exactly nothing: out = fma(U, 1/l, 0) is the plain product."""
    cfg = ATTN_CFGS[name]
    geom, tab, x = _setup(cfg)
    gate = torch.zeros((cfg["h"], cfg["D"]), dtype=torch.float32, device=DEV)
    o1, i1, _ = bsa.vsa_forward(x["q"], x["k"], x["v"], geom, cfg["R"], gate=gate)
    o2, i2, _ = bsa.vsa_forward(x["q"], x["k"], x["v"], geom, cfg["R"])
    torch.cuda.synchronize()
    assert torch.equal(i1, i2)
    assert torch.equal(o1.float(), o2.float())


def test_coarse_with_summaries():
    """Spark-Reweight virtual tokens and the coarse branch in one call."""
    cfg = scaled("video", grid=(8, 24, 28), h=2, R=6)
    geom, tab, x = _setup(cfg)
    B, N, H, D = x["q"].shape
    J = geom.J
    idx, num = kept_lists(B, H, J, min(9, J), seed=32, device=DEV)
    Q, K, V = to64(x["q"]), to64(x["k"]), to64(x["v"])
    ks, vs, b, _ = oracle.block_summaries(K, V, tab["perm"], tab["block_len"], tab["M"], oracle.anchor_queries(Q))
    k_sum = torch.from_numpy(ks).to(DEV, torch.bfloat16).contiguous()
    v_sum = torch.from_numpy(vs).to(DEV, torch.bfloat16).contiguous()
    b_sum = torch.from_numpy(b).to(DEV, torch.float32).contiguous()
    E32 = _oracle_scores(Q, K, tab).astype(np.float32)
    gate = coarse_gate(H, D, seed=33, device=DEV)
    C = bsa.coarse_attention(x["v"], geom.perm, geom.block_len, J, geom.M, torch.from_numpy(E32).to(DEV))
    out, lse = bsa.attention_vsa(x["q"], x["k"], x["v"], geom.perm, geom.block_len, J, geom.M, idx, num,
                                 need_lse=True, summaries=(k_sum, v_sum, b_sum), coarse=(C, gate))
    torch.cuda.synchronize()
    O, LSE = oracle.reweight_attention(Q, K, V, tab["perm"], tab["block_len"], tab["M"], idx.cpu().numpy(),
                                       num.cpu().numpy(), to64(k_sum), to64(v_sum), to64(b_sum))
    rv = oracle.pool_blocks(V, tab["perm"], tab["block_len"], tab["M"])
    rC = oracle.coarse_attention(E32.astype(np.float64), rv)
    ref = oracle.add_coarse(O, rC, to64(gate), tab["perm"], tab["block_len"], tab["M"])
    assert_attn_close(out, ref, "summaries+coarse")
    # the branch leaves the log-sum-exp of the sparse softmax unchanged
    assert np.max(np.abs(to64(lse) - LSE)) < 1e-3


def test_coarse_argument_errors():
    cfg = scaled("video", grid=(4, 8, 8), h=2, R=2)
    geom, tab, x = _setup(cfg)
    B, N, H, D = x["q"].shape
    J = geom.J
    E = torch.zeros((B, H, J, J), dtype=torch.float32, device=DEV)
    with pytest.raises(ValueError):  # scores of the wrong size
        bsa.coarse_attention(x["v"], geom.perm, geom.block_len, J, geom.M, E[..., :-1].contiguous())
    v96 = torch.zeros((B, N, H, 96), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(bsa._lib.BsaError, match="D must be 64 or 128"):
        bsa.coarse_attention(v96, geom.perm, geom.block_len, J, geom.M, E)
    C = bsa.coarse_attention(x["v"], geom.perm, geom.block_len, J, geom.M, E)
    idx, num = kept_lists(B, H, J, 2, seed=34, device=DEV)
    gate_buf = torch.zeros(H * D + 1, dtype=torch.float32, device=DEV)
    gate = gate_buf[1:].view(H, D)  # contiguous, 4 bytes off a 16-byte boundary
    with pytest.raises(bsa._lib.BsaError, match="16-byte aligned"):
        bsa.attention_vsa(x["q"], x["k"], x["v"], geom.perm, geom.block_len, J, geom.M, idx, num,
                          coarse=(C, gate))
    with pytest.raises(ValueError):
        bsa.attention_vsa(x["q"], x["k"], x["v"], geom.perm, geom.block_len, J, geom.M, idx, num,
                          coarse=(C.to(torch.bfloat16), gate_buf[:H * D].view(H, D)))


def test_video_full_size_sampled():
    """The video workload at full size (115200 tokens, 24 heads, J = 1920,
    R = 192) with the gated branch, in the launch configuration of bench.py:
    C of three heads in full and the output on sampled query blocks of those
    heads against the oracle."""
    cfg = workload("video")
    geom, tab, x = _setup(cfg)
    B, N, H, D = x["q"].shape
    J = geom.J
    gate = coarse_gate(H, D, seed=35, device=DEV)
    print("video full size with the coarse branch, J", J, flush=True)
    E = torch.empty((B, H, J, J), dtype=torch.float32, device=DEV)
    order = torch.empty((B, H, J), dtype=torch.int32, device=DEV)
    idx, num = bsa.pool_route_topk(x["q"], x["k"], geom.perm, geom.block_len, J, geom.M, cfg["R"], scores=E,
                                   item_order=order)
    C = bsa.coarse_attention(x["v"], geom.perm, geom.block_len, J, geom.M, E)
    out = bsa.attention_vsa(x["q"], x["k"], x["v"], geom.perm, geom.block_len, J, geom.M, idx, num,
                            item_order=order, coarse=(C, gate))
    torch.cuda.synchronize()
    heads = [0, 11, 23]
    Q, K, V = (to64(t[:, :, heads]) for t in (x["q"], x["k"], x["v"]))
    rE = _oracle_scores(Q, K, tab)
    rv = oracle.pool_blocks(V, tab["perm"], tab["block_len"], tab["M"])
    rC = oracle.coarse_attention(rE, rv)
    dE = 2e-5 * max(1.0, float(np.abs(rE).max()))
    bound = _c_bound(rE, rv, V, J) + 2 * dE * float(np.abs(rv).max())
    err = float(np.max(np.abs(to64(C[:, heads]) - rC)))
    print("video C: max abs err %.3g (bound %.3g)" % (err, bound), flush=True)
    assert err <= bound
    rng = np.random.default_rng(36)
    blocks = [0, 1, J - 1] + [int(v) for v in rng.choice(J, 5, replace=False)]
    items = [(0, hi, i) for hi in range(len(heads)) for i in blocks]
    hsel = torch.tensor(heads, device=DEV)
    O, _ = oracle.vsa_attention(Q, K, V, tab["perm"], tab["block_len"], tab["M"], idx[:, hsel].cpu().numpy(),
                                num[:, hsel].cpu().numpy(), items=items)
    ref = oracle.add_coarse(O, rC, to64(gate[hsel]), tab["perm"], tab["block_len"], tab["M"])
    got = to64(out[:, :, heads])
    mask = ~np.isnan(ref)
    assert_attn_close(got[mask], ref[mask], "video full size, sampled blocks with the coarse branch")


def test_coarse_is_deterministic():
    """Two launches on the same scores give the same C bit for bit."""
    cfg = COARSE_CFGS["odd_two_chunks"]
    geom, tab, x = _setup(cfg)
    J = geom.J
    Q, K = to64(x["q"]), to64(x["k"])
    E = torch.from_numpy(_oracle_scores(Q, K, tab).astype(np.float32)).to(DEV).contiguous()
    C1 = bsa.coarse_attention(x["v"], geom.perm, geom.block_len, J, geom.M, E)
    C2 = bsa.coarse_attention(x["v"], geom.perm, geom.block_len, J, geom.M, E)
    torch.cuda.synchronize()
    assert torch.equal(C1, C2)
